// Internal kernel launchers (host side), one per step of the path. The
// public C ABI in api.hip validates arguments and calls these.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

hipError_t launch_route(const float* logits, long T, long ld, int n_routed,
                        int n_sink, int k, float scale, int* ids, float* w,
                        float* sw, hipStream_t s);

// permute: rank/count, scan, scatter (three launches)
constexpr int kPermBlock = 1024;
size_t permute_ws_bytes(long T, int k, int G);
hipError_t launch_permute(const int* ids, long T, int k, int E_global, int off,
                          int E_loc, int shared, int* offsets,
                          int* sorted_pair, int* pair_row, int* err_word,
                          void* ws, hipStream_t s);

hipError_t launch_quant_act(const void* x, long T, int H, void* xq, float* xs,
                            hipStream_t s);

// z[r][q] = sum_h x[t(r)][h] * A[g(r)][q][h] for every sorted row of a
// local group (fp32)
hipError_t launch_lora_z(const void* x_bf16, const void* A, int rank, long T,
                         int H, int top_k, int n_lora_groups, long p_cap,
                         const int* offsets, const int* sorted_pair, float* z,
                         hipStream_t s);

// Stream-K for the FP8 grouped GEMMs at decode sizes: considered when at
// most kSkMaxTiles tiles can exist (tiles <= min(p_cap, G + p_cap / 32) *
// NT, NS K blocks each) and chosen when one tile per workgroup, in waves
// over an MI355X's kSkCUs CUs, would leave idle slots worth 8 or more K
// blocks per CU. The decision depends on the shapes only (workspace sizes
// are computed without a device); the partial sums then need kSkSlots *
// p_cap * N fp32 of workspace.
constexpr long kSkMaxTiles = 1024;
constexpr long kSkCUs = 256;
constexpr int kSkSlots = 4;          // partial-sum slots per tile
constexpr int kSkBM = 32;            // tile rows under stream-K
bool fp8_streamk(int fmt, long p_cap, int G, int NT, int NS);

struct Gemm1Args {
  int fmt;
  const void* wq;
  const void* ws;
  const float* gscale;
  const void* x;
  const float* xs;
  long T;
  int H, I, top_k, G;
  long p_cap;
  const int* offsets;
  const int* sorted_pair;
  float alpha, beta, limit;
  const float* z;        // LoRA z rows [p_cap][rank] or NULL
  const void* lora_B;    // bf16 [E_loc][2I][rank]
  int lora_rank, lora_groups;
  float lora_scale;
  void* h;
  float* hs;
  float* part;           // stream-K partials (when fp8_streamk) or NULL
};
hipError_t launch_gemm1(const Gemm1Args& a, hipStream_t s);

struct Gemm2Args {
  int fmt;
  const void* wq;
  const void* ws;
  const void* h;
  const float* hs;
  int H, I, G;
  long p_cap;
  const int* offsets;
  float* y;              // [p_cap][H] fp32, or the stream-K partials
  int* sk_grid;          // out: stream-K workgroup count (0 = plain y)
};
hipError_t launch_gemm2(const Gemm2Args& a, hipStream_t s);

// sk_grid > 0: y holds stream-K partials of the FP8 GEMM2 over G groups,
// reduced here per element in slot order
hipError_t launch_combine(const float* y, long T, int H, int top_k, int shared,
                          const int* pair_row, const float* topk_w,
                          float shared_w, float* out, hipStream_t s,
                          int sk_grid = 0, long p_cap = 0, int I = 0, int G = 0,
                          const int* offsets = nullptr);

}  // namespace moe
