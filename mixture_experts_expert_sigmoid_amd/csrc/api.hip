// Host side of the C ABI (include/moe_mi355x.h): argument validation,
// workspace carving and kernel launches. No allocation, no synchronisation
// (except moe_read_device_error), no state kept between calls apart from the
// calling thread's last HIP error message.
#include <math.h>

#include <algorithm>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "common.h"
#include "launch.h"
#include "moe_mi355x.h"

static_assert(MOE_DEVERR_GLOBAL_ID_OOB == MOE_DEVERR_BIT_OOB, "err bit");
static_assert(MOE_DEVERR_F16_RANGE == MOE_DEVERR_BIT_F16_RANGE, "err bit");
static_assert(MOE_DEVERR_W4_SCALE == MOE_DEVERR_BIT_W4_SCALE, "err bit");

namespace {

thread_local char g_last_error[256] = "";

int hip_fail(hipError_t e, const char* where) {
  snprintf(g_last_error, sizeof g_last_error, "%s: %s", where,
           hipGetErrorString(e));
  return MOE_ERR_HIP;
}

inline size_t al(size_t b) { return (b + 255) & ~(size_t)255; }
constexpr int kMaxAdapters = 1024;
inline bool finite(float v) { return isfinite(v); }

// 4-bit formats: packed codes, the 4-bit kernel family, bf16 h
bool is4(int fmt) {
  return fmt == MOE_W_INT4_G32 || fmt == MOE_W_NVFP4 || fmt == MOE_W_MXFP4 ||
         fmt == MOE_W_MXFP4_A8;
}
bool is_fp4(int fmt) {
  return fmt == MOE_W_NVFP4 || fmt == MOE_W_MXFP4 || fmt == MOE_W_MXFP4_A8;
}
// GEMM1 takes quantised activation codes with scales (FP8, MXFP8)
bool quant_act(int fmt) { return fmt == MOE_W_FP8_B128 || fmt == MOE_W_MXFP4_A8; }

// w2: the down weight, whose global scales ([G]) only FP4 formats take
int check_weights(const moe_weights* w, int N, int K, bool w2 = false) {
  if (!w || !w->q) return MOE_ERR_NULL;
  if (w->fmt < MOE_W_BF16 || w->fmt > MOE_W_MXFP4_A8) return MOE_ERR_FORMAT;
  if (w->fmt != MOE_W_BF16 && !w->scale) return MOE_ERR_NULL;
  if (w2 && w->gscale && !is_fp4(w->fmt)) return MOE_ERR_FORMAT;
  if (w->N != N || w->K != K) return MOE_ERR_SHAPE;
  if (w->n_groups < 1 || w->n_groups > 1024) return MOE_ERR_SHAPE;
  // 16-byte code loads; 2-byte scale words (INT4 bf16, NVFP4 e4m3 pairs)
  if (is4(w->fmt) && ((uintptr_t)w->q & 15)) return MOE_ERR_PARAM;
  if ((w->fmt == MOE_W_INT4_G32 || w->fmt == MOE_W_NVFP4) && ((uintptr_t)w->scale & 1))
    return MOE_ERR_PARAM;
  return MOE_OK;
}

int check_act(const moe_act_params* a) {
  if (!a) return MOE_ERR_NULL;
  if (!finite(a->alpha) || !finite(a->beta) || !(a->limit > 0.0f))
    return MOE_ERR_PARAM;
  return MOE_OK;
}

int check_lora(const moe_lora* l, int G) {
  if (!l) return MOE_OK;
  if (!l->A || !l->B) return MOE_ERR_NULL;
  if (l->rank < 1 || l->rank > 32) return MOE_ERR_SHAPE;
  if (l->n_groups < 0 || l->n_groups > G) return MOE_ERR_SHAPE;
  if (!finite(l->scale)) return MOE_ERR_PARAM;
  if (l->n_adapters < 0 || l->n_adapters > kMaxAdapters) return MOE_ERR_SHAPE;
  if (l->n_adapters > 1 && !l->adapter_ids) return MOE_ERR_NULL;
  if ((((uintptr_t)l->A) | ((uintptr_t)l->B)) & 15) return MOE_ERR_PARAM;   // 16-byte loads
  return MOE_OK;
}

bool batched(const moe_lora* l) { return l && l->n_adapters > 1; }

long pcap_of(long T, int k, int shared) { return T * (long)k + (shared ? T : 0); }

}  // namespace

extern "C" {

const char* moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "required pointer is NULL";
    case MOE_ERR_SHAPE: return "size out of range or not a required multiple";
    case MOE_ERR_FORMAT: return "unknown or mismatched weight format";
    case MOE_ERR_LOCAL_RANGE: return "missing or invalid local expert range";
    case MOE_ERR_PARAM: return "non-finite or out-of-range parameter";
    case MOE_ERR_WORKSPACE: return "workspace NULL or too small";
    case MOE_ERR_HIP: return "HIP launch or runtime failure";
    case MOE_ERR_SCRATCH: return "the call needs more than the static scratch holds";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_last_error; }

int moe_route(const float* logits, long T, long ld, int n_routed, int n_sink,
              int top_k, const float* sel_bias, float route_scale,
              float global_scale, int* topk_ids, float* topk_w, float* sink_w,
              int* packed, void* stream) {
  if (T < 0 || n_routed < 1 || n_sink < 0 || top_k < 1 || top_k > n_routed ||
      top_k + n_sink > 64 || n_routed + n_sink > 1024 || ld < n_routed + n_sink)
    return MOE_ERR_SHAPE;
  if (!finite(route_scale) || !finite(global_scale)) return MOE_ERR_PARAM;
  if (T > 0 && (!logits || !topk_ids || !topk_w || (n_sink > 0 && !sink_w)))
    return MOE_ERR_NULL;
  hipError_t e = moe::launch_route(logits, T, ld, n_routed, n_sink, top_k,
                                   sel_bias, route_scale * global_scale,
                                   topk_ids, topk_w, sink_w, packed,
                                   (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route");
}

static int gate_checks(long T, int H, int n_routed, int n_sink, int top_k) {
  if (T < 0 || H < 32 || H % 32 != 0 || n_routed < 1 || n_sink < 0 ||
      top_k < 1 || top_k > n_routed || top_k + n_sink > 16 ||
      n_routed + n_sink > 512)
    return MOE_ERR_SHAPE;
  return MOE_OK;
}

size_t moe_gate_route_workspace_size(long T, int H, int n_routed, int n_sink) {
  if (gate_checks(T, H, n_routed, n_sink, 1) != MOE_OK) return 0;
  return moe::gate_ws_bytes(T, H, n_routed + n_sink);
}

int moe_gate_route(const void* x_bf16, const void* wg_bf16, long T, int H,
                   int n_routed, int n_sink, int top_k, const float* sel_bias,
                   float route_scale, float global_scale, float* logits,
                   int* topk_ids, float* topk_w, float* sink_w, int* packed,
                   void* ws, size_t ws_bytes, void* stream) {
  int st = gate_checks(T, H, n_routed, n_sink, top_k);
  if (st) return st;
  if (!finite(route_scale) || !finite(global_scale)) return MOE_ERR_PARAM;
  if (T > 0 && (!x_bf16 || !wg_bf16 || !topk_ids || !topk_w ||
                (n_sink > 0 && !sink_w)))
    return MOE_ERR_NULL;
  if ((((uintptr_t)x_bf16) | ((uintptr_t)wg_bf16)) & 15) return MOE_ERR_PARAM;
  const size_t need = moe::gate_ws_bytes(T, H, n_routed + n_sink);
  if (need > 0 && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  moe::GateArgs a{};
  a.x = x_bf16;
  a.wg = wg_bf16;
  a.T = T;
  a.H = H;
  a.n_routed = n_routed;
  a.n_sink = n_sink;
  a.k = top_k;
  a.bias = sel_bias;
  a.scale = route_scale * global_scale;
  a.logits = logits;
  a.ids = topk_ids;
  a.w = topk_w;
  a.sw = sink_w;
  a.packed = packed;
  a.ws = ws;
  hipError_t e = moe::launch_gate(a, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_gate_route");
}

size_t moe_permute_workspace_size(long T, int top_k, int n_groups) {
  if (T < 0 || top_k < 1 || n_groups < 1) return 0;
  return moe::permute_ws_bytes(T, top_k, n_groups);
}

static int permute_checks(long T, int top_k, int E, int off, int E_loc,
                          int shared) {
  if (T < 0 || top_k < 1) return MOE_ERR_SHAPE;
  if (E_loc < 1 || off < 0 || (long)off + E_loc > E) return MOE_ERR_LOCAL_RANGE;
  if (shared != 0 && shared != 1) return MOE_ERR_PARAM;
  if (E_loc + shared > 1024) return MOE_ERR_SHAPE;
  if (T * (long)top_k >= (1L << 30)) return MOE_ERR_SHAPE;
  return MOE_OK;
}

int moe_permute(const int* topk_ids, long T, int top_k, int num_experts_global,
                int local_expert_offset, int num_local_experts,
                int shared_expert, int* offsets, int* sorted_pair,
                int* pair_row, int* err_word, void* ws, size_t ws_bytes,
                void* stream) {
  int st = permute_checks(T, top_k, num_experts_global, local_expert_offset,
                          num_local_experts, shared_expert);
  if (st) return st;
  long np = pcap_of(T, top_k, shared_expert);
  if (!offsets || !err_word || (T > 0 && !topk_ids) ||
      (np > 0 && (!sorted_pair || !pair_row)))
    return MOE_ERR_NULL;
  int G = num_local_experts + shared_expert;
  if (!ws || ws_bytes < moe::permute_ws_bytes(T, top_k, G))
    return MOE_ERR_WORKSPACE;
  hipError_t e = moe::launch_permute(
      topk_ids, T, top_k, num_experts_global, local_expert_offset,
      num_local_experts, shared_expert, offsets, sorted_pair, pair_row,
      err_word, ws, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_permute");
}

int moe_quantize_act_fp8(const void* x_bf16, long T, int H, void* xq,
                         float* xs, void* stream) {
  if (T < 0 || H < 128 || H % 128) return MOE_ERR_SHAPE;
  if (T > 0 && (!x_bf16 || !xq || !xs)) return MOE_ERR_NULL;
  hipError_t e = moe::launch_quant_act(x_bf16, T, H, xq, xs, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_quantize_act_fp8");
}

int moe_quantize_act_mxfp8(const void* x_bf16, long T, int H, void* xq, void* xe,
                           void* stream) {
  if (T < 0 || H < 128 || H % 128) return MOE_ERR_SHAPE;
  if (T > 0 && (!x_bf16 || !xq || !xe)) return MOE_ERR_NULL;
  hipError_t e = moe::launch_quant_act_mx(x_bf16, T, H, xq, xe, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_quantize_act_mxfp8");
}

}  // extern "C"

namespace {
// GEMM1 workspace: LoRA z rows, then (split-K) the fp32 partial sums, then
// (4-bit formats) the f16 activations, T <= p_cap rows of K
// LoRA z rows, and with a batch of adapters each row's adapter
size_t g1_z_bytes(long p_cap, const moe_lora* lora) {
  if (!lora) return 0;
  return al((size_t)p_cap * lora->rank * 4) + (batched(lora) ? al((size_t)p_cap * 4) : 0);
}
int* zad_of(float* z, long p_cap, const moe_lora* lora) {
  return batched(lora) ? (int*)((char*)z + al((size_t)p_cap * lora->rank * 4)) : nullptr;
}
size_t g1_part_bytes(const moe_weights* w13, long p_cap) {
  if (!moe::splitk_use(w13->fmt, p_cap, w13->n_groups, w13->N / 256, w13->K / 128, true))
    return 0;
  return moe::splitk_bytes(p_cap, w13->N);
}
size_t g1_x16_bytes(const moe_weights* w13, long rows) {
  return is4(w13->fmt) && w13->fmt != MOE_W_MXFP4_A8 ? al((size_t)rows * w13->K * 2) : 0;
}
// GEMM2 workspace: the y rows (fp32 for BF16 layers; int16 + one scale
// exponent per 16 columns otherwise, at most the fp32 size), or (split-K)
// their partial sums
size_t g2_bytes(const moe_weights* w2, long p_cap) {
  if (moe::splitk_use(w2->fmt, p_cap, w2->n_groups, (w2->N + 255) / 256, w2->K / 128, false))
    return moe::splitk_bytes(p_cap, w2->N);
  return al((size_t)p_cap * w2->N * 4);
}
}  // namespace

extern "C" {

size_t moe_gemm1_workspace_size(const moe_weights* w13, long p_cap,
                                const moe_lora* lora) {
  if (!w13 || p_cap < 0 || w13->N < 256 || w13->N % 256) return 0;
  return g1_z_bytes(p_cap, lora) + g1_part_bytes(w13, p_cap) + g1_x16_bytes(w13, p_cap);
}

static int gemm1_checks(const moe_weights* w13, const void* x, const void* xs,
                        const void* x_bf16, long T, int H, int I, int top_k,
                        long p_cap, const int* offsets, const int* sorted_pair,
                        const moe_act_params* act, const moe_lora* lora,
                        const void* h, const float* hs) {
  if (T < 0 || p_cap < 0 || top_k < 1) return MOE_ERR_SHAPE;
  if (H < 128 || I < 128 || H % 128 || I % 128) return MOE_ERR_SHAPE;
  int st = check_weights(w13, 2 * I, H);
  if (st) return st;
  if ((st = check_act(act))) return st;
  if ((st = check_lora(lora, w13->n_groups))) return st;
  if (!offsets || (p_cap > 0 && (!x || !sorted_pair || !h))) return MOE_ERR_NULL;
  if (w13->fmt == MOE_W_FP8_B128 && p_cap > 0 && (!xs || !hs)) return MOE_ERR_NULL;
  if (w13->fmt == MOE_W_MXFP4_A8 && p_cap > 0 && !xs) return MOE_ERR_NULL;
  if (lora && p_cap > 0 && !x_bf16) return MOE_ERR_NULL;
  return MOE_OK;
}

static moe::Gemm1Args gemm1_args(const moe_weights* w13, const void* x,
                                 const void* xs, long T, int H, int I,
                                 int top_k, long p_cap, const int* offsets,
                                 const int* sorted_pair,
                                 const moe_act_params* act,
                                 const moe_lora* lora, const float* z, void* h,
                                 float* hs, float* part, void* x16, void* h_lora,
                                 int* err_word) {
  moe::Gemm1Args a{};
  a.fmt = w13->fmt;
  a.wq = w13->q;
  a.ws = w13->scale;
  a.gscale = w13->gscale;
  a.x = x;
  a.xs = xs;
  a.T = T;
  a.H = H;
  a.I = I;
  a.top_k = top_k;
  a.G = w13->n_groups;
  a.p_cap = p_cap;
  a.offsets = offsets;
  a.sorted_pair = sorted_pair;
  a.alpha = act->alpha;
  a.beta = act->beta;
  a.limit = act->limit;
  a.z = lora ? z : nullptr;
  a.lora_B = lora ? lora->B : nullptr;
  a.lora_rank = lora ? lora->rank : 0;
  a.lora_groups = lora ? lora->n_groups : 0;
  a.lora_scale = lora ? lora->scale : 0.0f;
  a.n_adapters = lora ? lora->n_adapters : 0;
  a.zad = lora ? zad_of(const_cast<float*>(z), p_cap, lora) : nullptr;
  a.h = h;
  a.hs = hs;
  a.part = part;
  a.x16 = x16;
  a.h_lora = h_lora;
  a.err = err_word;
  return a;
}

int moe_grouped_gemm1_act(const moe_weights* w13, const void* x,
                          const void* xs, const void* x_bf16, long T, int H,
                          int I, int top_k, long p_cap, const int* offsets,
                          const int* sorted_pair, const moe_act_params* act,
                          const moe_lora* lora, void* h, float* hs, void* h_lora,
                          int* err_word, void* ws, size_t ws_bytes, void* stream) {
  int st = gemm1_checks(w13, x, xs, x_bf16, T, H, I, top_k, p_cap, offsets,
                        sorted_pair, act, lora, h, hs);
  if (st) return st;
  // 4-bit layers report activation and scale range problems there
  if (is4(w13->fmt) && p_cap > 0 && !err_word) return MOE_ERR_NULL;
  // BF16 / 4-bit layers write h in bf16 already: it is the down-LoRA input
  if (h_lora && w13->fmt != MOE_W_FP8_B128) return MOE_ERR_PARAM;
  size_t need = moe_gemm1_workspace_size(w13, p_cap, lora);
  if (need && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (is4(w13->fmt) && T > p_cap) return MOE_ERR_SHAPE;
  float* z = (float*)ws;
  float* part = g1_part_bytes(w13, p_cap)
                    ? (float*)((char*)ws + g1_z_bytes(p_cap, lora)) : nullptr;
  void* x16 = (char*)ws + g1_z_bytes(p_cap, lora) + g1_part_bytes(w13, p_cap);
  hipError_t e = hipSuccess;
  if (lora)
    e = moe::launch_lora_z(x_bf16, lora->A, lora->rank, T, H, top_k,
                           lora->n_groups, p_cap, offsets, sorted_pair, true,
                           lora->n_adapters, lora->adapter_ids, z,
                           zad_of(z, p_cap, lora), s);
  if (e == hipSuccess)
    e = moe::launch_gemm1(gemm1_args(w13, x, xs, T, H, I, top_k, p_cap, offsets,
                                     sorted_pair, act, lora, z, h, hs, part, x16,
                                     h_lora, err_word), s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_grouped_gemm1_act");
}

size_t moe_gemm2_workspace_size(const moe_weights* w2, long p_cap,
                                const moe_lora* lora_down) {
  if (!w2 || p_cap < 0 || w2->N < 0) return 0;
  return g2_bytes(w2, p_cap) + g1_z_bytes(p_cap, lora_down);
}

static int gemm2_checks(const moe_weights* w2, const void* h, const float* hs,
                        long T, int H, int I, int top_k, int shared,
                        long p_cap, const int* offsets, const int* pair_row,
                        const float* topk_w, float shared_w, const float* out) {
  // top_k <= 64: the split-K combine keeps a token's top_k + 1 pairs in LDS
  if (T < 0 || p_cap < 0 || top_k < 1 || top_k > 64) return MOE_ERR_SHAPE;
  if (H < 128 || I < 128 || H % 128 || I % 128) return MOE_ERR_SHAPE;
  if (shared != 0 && shared != 1) return MOE_ERR_PARAM;
  if (!finite(shared_w)) return MOE_ERR_PARAM;
  int st = check_weights(w2, H, I, true);
  if (st) return st;
  if (!offsets) return MOE_ERR_NULL;
  if (p_cap > 0 && (!h || (w2->fmt == MOE_W_FP8_B128 && !hs))) return MOE_ERR_NULL;
  if (T > 0 && (!out || !pair_row || !topk_w)) return MOE_ERR_NULL;
  if (p_cap < pcap_of(T, top_k, shared) && T > 0) return MOE_ERR_SHAPE;
  return MOE_OK;
}

int moe_grouped_gemm2_combine(const moe_weights* w2, const void* h,
                              const float* hs, const void* h_lora,
                              const moe_lora* lora_down, long T, int H, int I,
                              int top_k, int shared_expert, long p_cap,
                              const int* offsets, const int* sorted_pair,
                              const int* pair_row, const float* topk_w,
                              float shared_w, float* out, int* err_word, void* ws,
                              size_t ws_bytes, void* stream) {
  int st = gemm2_checks(w2, h, hs, T, H, I, top_k, shared_expert, p_cap,
                        offsets, pair_row, topk_w, shared_w, out);
  if (st) return st;
  if (is4(w2->fmt) && p_cap > 0 && !err_word) return MOE_ERR_NULL;
  if ((st = check_lora(lora_down, w2->n_groups))) return st;
  if (lora_down && p_cap > 0 && (!h_lora || !sorted_pair)) return MOE_ERR_NULL;
  size_t need = moe_gemm2_workspace_size(w2, p_cap, lora_down);
  if (need && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  float* y = (float*)ws;
  float* z2 = (float*)((char*)ws + g2_bytes(w2, p_cap));
  hipError_t e = hipSuccess;
  if (lora_down)
    e = moe::launch_lora_z(h_lora, lora_down->A, lora_down->rank, T, I, top_k,
                           lora_down->n_groups, p_cap, offsets, sorted_pair, false,
                           lora_down->n_adapters, lora_down->adapter_ids, z2,
                           zad_of(z2, p_cap, lora_down), s);
  if (e != hipSuccess) return hip_fail(e, "moe_grouped_gemm2_combine/lora_z");
  moe::Gemm2Args a{};
  a.fmt = w2->fmt;
  a.wq = w2->q;
  a.ws = w2->scale;
  a.gscale = w2->gscale;
  a.h = h;
  a.hs = hs;
  a.H = H;
  a.I = I;
  a.G = w2->n_groups;
  a.p_cap = p_cap;
  a.offsets = offsets;
  a.y = y;
  int sk_grid = 0, sk_mode = 0;
  a.sk_grid = &sk_grid;
  a.sk_mode = &sk_mode;
  if (lora_down) {
    a.z = z2;
    a.lora_B = lora_down->B;
    a.lora_rank = lora_down->rank;
    a.lora_groups = lora_down->n_groups;
    a.lora_scale = lora_down->scale;
    a.n_adapters = lora_down->n_adapters;
    a.zad = zad_of(z2, p_cap, lora_down);
  }
  a.err = err_word;
  e = moe::launch_gemm2(a, s);
  if (e == hipSuccess)
    e = moe::launch_combine(y, T, H, top_k, shared_expert, pair_row, topk_w,
                            shared_w, out, s, sk_grid, p_cap, I, a.G, offsets, sk_mode,
                            w2->fmt != MOE_W_BF16);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_grouped_gemm2_combine");
}

// ---------------------------------------------------------------- forward --

namespace {
struct FwdLayout {
  size_t offsets, sorted_pair, pair_row, perm_ws, xq, xs, z, h, hs, h_lora, z2, y, total;
  size_t perm_bytes;
};

FwdLayout layout(const moe_layer* L, long T) {
  FwdLayout o{};
  int G = L->num_local_experts + L->shared_expert;
  long pc = pcap_of(T, L->top_k, L->shared_expert);
  bool fp8 = L->w13.fmt == MOE_W_FP8_B128;
  bool mx = L->w13.fmt == MOE_W_MXFP4_A8;
  size_t cur = 0;
  auto take = [&](size_t bytes) { size_t at = cur; cur += al(bytes); return at; };
  o.offsets = take((size_t)(G + 1) * 4);
  o.sorted_pair = take((size_t)pc * 4);
  o.pair_row = take((size_t)pc * 4);
  o.perm_bytes = moe::permute_ws_bytes(T, L->top_k, G);
  o.perm_ws = take(o.perm_bytes);
  // FP8 / MXFP8 activation codes, or (other 4-bit formats) the f16 activations
  o.xq = take(fp8 || mx ? (size_t)T * L->H : g1_x16_bytes(&L->w13, T));
  o.xs = take(fp8 ? (size_t)T * (L->H / 128) * 4 : mx ? (size_t)T * (L->H / 32) : 0);
  o.z = take(g1_z_bytes(pc, L->lora));
  o.h = take((size_t)pc * L->I * (fp8 ? 1 : 2));
  o.hs = take(fp8 ? (size_t)pc * (L->I / 128) * 4 : 0);
  // down LoRA: its bf16 input (FP8 layers; BF16 / 4-bit layers read h) and z rows
  o.h_lora = take(fp8 && L->lora_down ? (size_t)pc * L->I * 2 : 0);
  o.z2 = take(g1_z_bytes(pc, L->lora_down));
  // y rows (or their stream-K partials); GEMM1's partials, consumed before
  // GEMM2 starts, share the region
  o.y = take(std::max(g2_bytes(&L->w2, pc), g1_part_bytes(&L->w13, pc)));
  o.total = cur;
  return o;
}

int layer_checks(const moe_layer* L) {
  if (!L) return MOE_ERR_NULL;
  if (L->H < 128 || L->I < 128 || L->H % 128 || L->I % 128) return MOE_ERR_SHAPE;
  int st = permute_checks(0, L->top_k, L->num_experts_global,
                          L->local_expert_offset, L->num_local_experts,
                          L->shared_expert);
  if (st) return st;
  int G = L->num_local_experts + L->shared_expert;
  if ((st = check_weights(&L->w13, 2 * L->I, L->H))) return st;
  if ((st = check_weights(&L->w2, L->H, L->I, true))) return st;
  if (L->w13.n_groups != G || L->w2.n_groups != G) return MOE_ERR_SHAPE;
  if (L->w13.fmt != L->w2.fmt) return MOE_ERR_FORMAT;
  if ((st = check_act(&L->act))) return st;
  if ((st = check_lora(L->lora, G))) return st;
  if (L->lora && L->lora->n_groups > L->num_local_experts) return MOE_ERR_SHAPE;
  if ((st = check_lora(L->lora_down, G))) return st;
  if (L->lora_down && L->lora_down->n_groups > L->num_local_experts) return MOE_ERR_SHAPE;
  if (L->n_sink < 0 || L->top_k > L->num_experts_global ||
      L->top_k + L->n_sink > 64 || L->num_experts_global + L->n_sink > 1024)
    return MOE_ERR_SHAPE;
  if (!finite(L->route_scale) || !finite(L->global_scale) || !finite(L->shared_w))
    return MOE_ERR_PARAM;
  return MOE_OK;
}
}  // namespace

size_t moe_workspace_size(const moe_layer* layer, long T_max) {
  if (!layer || T_max < 0 || layer_checks(layer) != MOE_OK) return 0;
  return layout(layer, T_max).total;
}

int moe_forward(const moe_layer* L, const void* x_bf16, const float* logits,
                long T, long ld_logits, float* out, int* topk_ids,
                float* topk_w, float* sink_w, int* err_word, void* ws,
                size_t ws_bytes, void* stream) {
  int st = layer_checks(L);
  if (st) return st;
  if (T < 0) return MOE_ERR_SHAPE;
  if (ld_logits < L->num_experts_global + L->n_sink) return MOE_ERR_SHAPE;
  if (!err_word) return MOE_ERR_NULL;
  if (T > 0 && (!x_bf16 || !logits || !out || !topk_ids || !topk_w ||
                (L->n_sink > 0 && !sink_w)))
    return MOE_ERR_NULL;
  if (T * (long)L->top_k >= (1L << 30)) return MOE_ERR_SHAPE;
  FwdLayout o = layout(L, T);
  if (!ws || ws_bytes < o.total) return MOE_ERR_WORKSPACE;
  char* base = (char*)ws;
  hipStream_t s = (hipStream_t)stream;
  const int G = L->num_local_experts + L->shared_expert;
  const long pc = pcap_of(T, L->top_k, L->shared_expert);
  int* offsets = (int*)(base + o.offsets);
  int* sorted_pair = (int*)(base + o.sorted_pair);
  int* pair_row = (int*)(base + o.pair_row);
  const bool fp8 = L->w13.fmt == MOE_W_FP8_B128;
  void* xq = base + o.xq;
  float* xs = (float*)(base + o.xs);
  float* z = (float*)(base + o.z);
  void* h = base + o.h;
  float* hs = (float*)(base + o.hs);
  float* y = (float*)(base + o.y);
  void* h_lora = fp8 ? (void*)(base + o.h_lora) : h;
  float* z2 = (float*)(base + o.z2);

  const bool four = is4(L->w13.fmt);
  const bool mx = L->w13.fmt == MOE_W_MXFP4_A8;
  bool x16_ready = false;
  hipError_t e = hipSuccess;
  const bool small = moe::front_small_fits(T, L->top_k, G, L->H);
  {
    // decode sizes: route + activation pass + permute in one launch; larger
    // batches: route + activation pass in one launch, then the permutation
    moe::FrontArgs fa{};
    fa.logits = logits;
    fa.T = T;
    fa.ld = ld_logits;
    fa.n_routed = L->num_experts_global;
    fa.n_sink = L->n_sink;
    fa.k = L->top_k;
    fa.scale = L->route_scale * L->global_scale;
    fa.ids = topk_ids;
    fa.w = topk_w;
    fa.sw = sink_w;
    fa.x = x_bf16;
    fa.H = L->H;
    fa.xq = xq;
    fa.xs = xs;
    fa.off = L->local_expert_offset;
    fa.E_loc = L->num_local_experts;
    fa.G = G;
    fa.shared = L->shared_expert;
    fa.offsets = offsets;
    fa.sorted_pair = sorted_pair;
    fa.pair_row = pair_row;
    fa.err_word = err_word;
    const int mode = fp8 ? 1 : mx ? 3 : (four ? 2 : 0);
    e = small ? moe::launch_front_small(fa, mode, s) : moe::launch_front_large(fa, mode, s);
    if (e != hipSuccess) return hip_fail(e, "moe_forward/front");
    x16_ready = four && !mx;
  }
  if (!small) {
    e = moe::launch_permute(topk_ids, T, L->top_k, L->num_experts_global,
                            L->local_expert_offset, L->num_local_experts,
                            L->shared_expert, offsets, sorted_pair, pair_row,
                            err_word, base + o.perm_ws, s);
    if (e != hipSuccess) return hip_fail(e, "moe_forward/permute");
  }
  if (L->lora) {
    e = moe::launch_lora_z(x_bf16, L->lora->A, L->lora->rank, T, L->H,
                           L->top_k, L->lora->n_groups, pc, offsets,
                           sorted_pair, true, L->lora->n_adapters,
                           L->lora->adapter_ids, z, zad_of(z, pc, L->lora), s);
    if (e != hipSuccess) return hip_fail(e, "moe_forward/lora_z");
  }
  float* g1_part = g1_part_bytes(&L->w13, pc) ? y : nullptr;
  moe::Gemm1Args ga = gemm1_args(&L->w13, fp8 || mx ? xq : x_bf16,
                                 fp8 || mx ? (const void*)xs : nullptr,
                                 T, L->H, L->I, L->top_k, pc, offsets,
                                 sorted_pair, &L->act, L->lora, z, h,
                                 fp8 ? hs : nullptr, g1_part, xq,
                                 fp8 && L->lora_down ? h_lora : nullptr, err_word);
  ga.x16_ready = x16_ready;
  e = moe::launch_gemm1(ga, s);
  if (e != hipSuccess) return hip_fail(e, "moe_forward/gemm1");
  if (L->lora_down) {
    e = moe::launch_lora_z(h_lora, L->lora_down->A, L->lora_down->rank, T, L->I,
                           L->top_k, L->lora_down->n_groups, pc, offsets,
                           sorted_pair, false, L->lora_down->n_adapters,
                           L->lora_down->adapter_ids, z2,
                           zad_of(z2, pc, L->lora_down), s);
    if (e != hipSuccess) return hip_fail(e, "moe_forward/lora_z_down");
  }
  moe::Gemm2Args a{};
  a.fmt = L->w2.fmt;
  a.wq = L->w2.q;
  a.ws = L->w2.scale;
  a.gscale = L->w2.gscale;
  a.h = h;
  a.hs = fp8 ? hs : nullptr;
  a.H = L->H;
  a.I = L->I;
  a.G = G;
  a.p_cap = pc;
  a.offsets = offsets;
  a.y = y;
  int sk_grid = 0, sk_mode = 0;
  a.sk_grid = &sk_grid;
  a.sk_mode = &sk_mode;
  if (L->lora_down) {
    a.z = z2;
    a.lora_B = L->lora_down->B;
    a.lora_rank = L->lora_down->rank;
    a.lora_groups = L->lora_down->n_groups;
    a.lora_scale = L->lora_down->scale;
    a.n_adapters = L->lora_down->n_adapters;
    a.zad = zad_of(z2, pc, L->lora_down);
  }
  a.err = err_word;
  e = moe::launch_gemm2(a, s);
  if (e != hipSuccess) return hip_fail(e, "moe_forward/gemm2");
  e = moe::launch_combine(y, T, L->H, L->top_k, L->shared_expert, pair_row,
                          topk_w, L->shared_w, out, s, sk_grid, pc, L->I, G, offsets, sk_mode,
                          L->w2.fmt != MOE_W_BF16);
  if (e != hipSuccess) return hip_fail(e, "moe_forward/combine");
  return MOE_OK;
}

int moe_read_device_error(const int* err_word, int* host_bits, void* stream) {
  if (!err_word || !host_bits) return MOE_ERR_NULL;
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e == hipSuccess)
    e = hipMemcpy(host_bits, err_word, sizeof(int), hipMemcpyDeviceToHost);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_read_device_error");
}

}  // extern "C"
