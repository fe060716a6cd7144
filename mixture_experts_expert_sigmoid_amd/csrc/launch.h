// Internal kernel launchers (host side), one per step of the path. The
// public C ABI in api.hip validates arguments and calls these.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// bias: NULL (rank on the raw logit) or [n_routed] (rank on fp32
// sigmoid(x) + bias); packed: NULL or [T][k] (id << 16 | bf16 weight)
hipError_t launch_route(const float* logits, long T, long ld, int n_routed,
                        int n_sink, int k, const float* bias, float scale,
                        int* ids, float* w, float* sw, int* packed,
                        hipStream_t s);

// Router GEMM fused with the gate epilogue. With at least kGateFusedTiles
// tiles of 32 tokens the GEMM and the epilogue run in one launch; below,
// the K range is split over about kGateSplitTarget / tiles workgroups per
// tile and the partial sums (workspace, gate_ws_bytes) are added by the
// epilogue kernel in split order.
constexpr long kGateFusedTiles = 96;
constexpr long kGateSplitTarget = 128;
struct GateArgs {
  const void* x;         // bf16 [T][H]
  const void* wg;        // bf16 [n_routed + n_sink][H]
  long T;
  int H, n_routed, n_sink, k;
  const float* bias;     // [n_routed] or NULL
  float scale;           // route_scale * global_scale
  float* logits;         // [T][n_routed + n_sink] or NULL
  int* ids;
  float* w;
  float* sw;
  int* packed;           // [T][k] or NULL
  void* ws;              // gate_ws_bytes(T, H, n_routed + n_sink) bytes
};
int gate_splits(long T, int H);
size_t gate_ws_bytes(long T, int H, int n_cols);
hipError_t launch_gate(const GateArgs& a, hipStream_t s);

// permute: rank/count, scan, scatter (three launches)
constexpr int kPermBlock = 1024;
size_t permute_ws_bytes(long T, int k, int G);
hipError_t launch_permute(const int* ids, long T, int k, int E_global, int off,
                          int E_loc, int shared, int* offsets,
                          int* sorted_pair, int* pair_row, int* err_word,
                          void* ws, hipStream_t s);

hipError_t launch_quant_act(const void* x, long T, int H, void* xq, float* xs,
                            hipStream_t s);
// MXFP8: x bf16 [T][H] -> e4m3 codes [T][H] + e8m0 codes [T][H/32]
hipError_t launch_quant_act_mx(const void* x, long T, int H, void* xq, void* xe,
                               hipStream_t s);

// Decode front end (front.hip): route (no bias, no packed output) + the
// activation pass + permute in one workgroup when T * k <= kPermBlock, 17 G
// ints fit 64 KB of LDS and T * ceil(H / 512) <= 64 (front_small_fits);
// hipErrorNotSupported otherwise. mode 1: FP8 quantisation into xq / xs; 2: the f16 copy of x
// into xq (4-bit formats); 3: MXFP8 quantisation into xq / xs (e8m0 bytes; the
// MXFP4 W4A8 format); 0: none.
struct FrontArgs {
  const float* logits;
  long T, ld;
  int n_routed, n_sink, k;
  float scale;
  int* ids;
  float* w;
  float* sw;
  const void* x;         // bf16 [T][H]
  int H;
  void* xq;
  void* xs;              // fp32 [T][H/128] (mode 1) or e8m0 [T][H/32] (mode 3)
  int off, E_loc, G, shared;
  int* offsets;
  int* sorted_pair;
  int* pair_row;
  int* err_word;
};
bool front_small_fits(long T, int k, int G, int H);
hipError_t launch_front_small(const FrontArgs& a, int mode, hipStream_t s);
// the router epilogue and the activation pass (mode as for the small front
// end) in one launch of independent workgroups, for any T; the permutation
// follows separately
hipError_t launch_front_large(const FrontArgs& a, int mode, hipStream_t s);

// z[r][q] = sum_h x[row][h] * A[a(r)][g(r)][q][h] for every sorted row r of
// a local group (fp32). row = t(r) = sorted_pair[r] / top_k when gather,
// else r itself (x then holds one row per sorted row, e.g. the down-LoRA
// input, and H is its length I). a(r) = adapter_ids[t(r)] with a batch of
// adapters (n_adapters > 1; none: z = 0), else 0; zad[r] (nullable) gets
// a(r), -1 for none.
hipError_t launch_lora_z(const void* x_bf16, const void* A, int rank, long T,
                         int H, int top_k, int n_lora_groups, long p_cap,
                         const int* offsets, const int* sorted_pair, bool gather,
                         int n_adapters, const int* adapter_ids, float* z,
                         int* zad, hipStream_t s);

// Split-K (stream-K) for the FP8 and 4-bit grouped GEMMs at decode sizes:
// used when at most kSkMaxTiles tiles of 32 rows can exist (tiles <=
// min(p_cap, G + p_cap / 32) * NT, NS K blocks each) and one tile per
// workgroup, in waves over an MI355X's kSkCUs CUs, would leave idle slots
// worth at least 8 K blocks per CU. A shape-only rule, so workspace sizes
// need no device; the partial sums need kSkSlots * p_cap * N fp32.
// For GEMM1, when that bound is too loose to decide because few rows per
// expert are possible (p_cap <= 16 G: skewed routing can leave far fewer
// tiles than the bound), the split-K kernel applies the same rule to the
// real tile count it reads from the expert offsets (SK_DEVICE) and runs
// whole tiles itself with the plain kernel's 32-row code when split-K does
// not pay; for NVFP4 and W4A8 with LoRA the plain kernel is launched as well
// and returns at once when split-K is chosen (and the split-K kernel when it
// is not). The reduction kernel decides the same way. GEMM2 (shorter K,
// smaller gains) keeps the shape-only rule.
constexpr long kSkMaxTiles = 1024;
constexpr long kSkCUs = 256;
constexpr int kSkSlots = 4;          // partial-sum slots per tile
constexpr int kSkBM = 32;            // tile rows under the split-K kernels
constexpr long kSkDeviceMaxTiles = 2048;   // bound on tiles for SK_DEVICE
enum { SK_PLAIN = 0, SK_SPLIT = 1, SK_DEVICE = 2 };
// g1: GEMM1 (SK_DEVICE allowed)
int splitk_mode(int fmt, long p_cap, int G, int NT, int NS, bool g1);
inline bool splitk_use(int fmt, long p_cap, int G, int NT, int NS, bool g1) {
  return splitk_mode(fmt, p_cap, G, NT, NS, g1) != SK_PLAIN;
}
// bytes of a split-K workspace (the partial-sum slots)
inline size_t splitk_bytes(long p_cap, int N) {
  return ((size_t)kSkSlots * p_cap * N * 4 + 255) & ~(size_t)255;
}

struct Gemm1Args {
  int fmt;
  const void* wq;
  const void* ws;
  const float* gscale;
  const void* x;
  const void* xs;        // FP8: fp32 [T][H/128]; MXFP4 W4A8: e8m0 [T][H/32]
  long T;
  int H, I, top_k, G;
  long p_cap;
  const int* offsets;
  const int* sorted_pair;
  float alpha, beta, limit;
  const float* z;        // LoRA z rows [p_cap][rank] or NULL
  const void* lora_B;    // bf16 [n_adapters][lora_groups][2I][rank]
  int lora_rank, lora_groups;
  float lora_scale;
  int n_adapters;        // > 1: a batch of adapters, row adapters in zad
  const int* zad;        // [p_cap] (a batch of adapters) or NULL
  void* h;
  float* hs;
  float* part;           // split-K partials (when splitk_use) or NULL
  void* x16;             // 4-bit formats: f16 activations (T * H * 2 bytes) or NULL
  bool x16_ready;        // x16 already holds them (the decode front end wrote it)
  void* h_lora;          // FP8: bf16 SwiGLU output before the requant, or NULL
  int* err;              // nullable: 4-bit range problems (f16 activations, scales)
};
hipError_t launch_gemm1(const Gemm1Args& a, hipStream_t s);

struct Gemm2Args {
  int fmt;
  const void* wq;
  const void* ws;
  const float* gscale;   // FP4 formats: [G] per-expert global scales, or NULL
  const void* h;
  const float* hs;
  int H, I, G;
  long p_cap;
  const int* offsets;
  float* y;              // [p_cap][H] fp32 (BF16), int16 rows + their scale
                         // exponents (FP8, 4-bit), or the split-K partials
  int* sk_grid;          // out: split-K kernel grid (0 = plain kernel)
  int* sk_mode;          // out: SK_PLAIN, SK_SPLIT or SK_DEVICE
  // down-projection LoRA (nullable z): y += scale * z[row] . B[a][g][n]
  const float* z;        // [p_cap][rank]
  const void* lora_B;    // bf16 [n_adapters][G_lora][H][rank]
  int lora_rank, lora_groups;
  float lora_scale;
  int n_adapters;
  const int* zad;
  int* err;              // nullable: 4-bit range problems (f16 h, scales)
};
hipError_t launch_gemm2(const Gemm2Args& a, hipStream_t s);

// sk_grid > 0: y holds the partial sums of the FP8 / 4-bit GEMM2's split-K
// kernel over G groups, reduced here per element in slot order (sk_mode
// SK_SPLIT), or -- SK_DEVICE -- either those or plain rows, as the device
// rule decides on the real tile count. sk_grid == 0: y holds GEMM2's rows,
// fp32 [p_cap][H] (y16 = false) or int16 [p_cap][H] followed by the int8
// scale exponents [p_cap][H / 16] (y16 = true, see store_y16)
hipError_t launch_combine(const float* y, long T, int H, int top_k, int shared,
                          const int* pair_row, const float* topk_w,
                          float shared_w, float* out, hipStream_t s,
                          int sk_grid = 0, long p_cap = 0, int I = 0, int G = 0,
                          const int* offsets = nullptr, int sk_mode = 0,
                          bool y16 = false);

}  // namespace moe
