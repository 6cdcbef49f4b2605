// Grouped MLP entry points: GroupedLinear(gate_up) -> ScaledSwiGLU -> GroupedLinear(down)
// and its backward, per "Efficient MoE Training for Biological Foundation Models",
// Challenge 3. Host code: argument checks, workspace carving, kernel sequencing on
// the caller's stream.
#include <cstring>
#include <string>

#include "common.h"
#include "gemm_bf16.h"
#include "gemm_f32.h"
#include "gemm_mx.h"
#include "internal.h"

namespace moe {

static bool is_act_ok(const moe_mlp_desc& d) {
  switch (d.compute) {
    case MOE_F32: return d.act == MOE_F32 && d.wt == MOE_F32;
    case MOE_BF16: return d.act == MOE_BF16 && d.wt == MOE_BF16;
    case MOE_MXFP8: return (d.act == MOE_BF16 || d.act == MOE_MXFP8) && (d.wt == MOE_BF16 || d.wt == MOE_MXFP8);
    case MOE_FP8: return (d.act == MOE_BF16 || d.act == MOE_FP8) && (d.wt == MOE_BF16 || d.wt == MOE_FP8);
  }
  return false;
}

moe_status validate_desc(const moe_mlp_desc& d, bool backward) {
  if (d.E < 1 || d.E > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID_ARG, "grouped MLP: E out of [1, 256]");
  if (d.H < 1 || d.I < 1) return fail(MOE_ERR_INVALID_ARG, "grouped MLP: H and I must be positive");
  if (d.compute != MOE_F32 && d.compute != MOE_BF16 && d.compute != MOE_MXFP8 && d.compute != MOE_FP8)
    return fail(MOE_ERR_INVALID_ARG, "grouped MLP: bad compute dtype");
  if (!is_act_ok(d)) return fail(MOE_ERR_INVALID_ARG, "grouped MLP: act/wt storage does not match compute dtype");
  if ((int64_t)d.H * d.I * 2 > 0x7FFFFFFFLL)
    return fail(MOE_ERR_UNSUPPORTED, "grouped MLP: one expert's weight exceeds 2^31 bytes");
  if (d.compute == MOE_BF16 || d.compute == MOE_MXFP8 || d.compute == MOE_FP8) {
    if (d.H % 256 != 0 || d.I % 128 != 0)
      return fail(MOE_ERR_UNSUPPORTED, "grouped MLP: bf16/fp8 kernels need H % 256 == 0 and I % 128 == 0");
    if (backward && d.I % 256 != 0)
      return fail(MOE_ERR_UNSUPPORTED, "grouped MLP backward: bf16 kernels need I % 256 == 0");
  }
  if (backward && d.compute == MOE_FP8 && d.act != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "grouped MLP backward: per-tensor FP8 takes bf16 activations (and bf16 master "
                                     "weights or weights packed by fp8_tensor_pack_weight_bwd)");
  if (backward && d.compute == MOE_MXFP8 && d.act != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "grouped MLP backward: MXFP8 takes bf16 activations (and bf16 master weights or "
                                     "weights packed by mxfp8_pack_weight_bwd)");
  return MOE_OK;
}

static size_t a256(size_t x) { return align_up(x, 256); }

size_t mlp_fwd_workspace_bytes(const moe_mlp_desc& d, int64_t R) {
  const size_t I = d.I, H = d.H, E = d.E;
  switch (d.compute) {
    case MOE_F32: return d.save_for_bwd ? 0 : a256(R * I * 4);
    case MOE_BF16: return (d.save_for_bwd ? 0 : a256(R * I * 2)) + grouped_gemm_workspace_bytes();
    case MOE_MXFP8: {
      size_t b = 0;
      // codes and step-major scales of what is given in bf16; converted scales otherwise
      b += (d.act == MOE_BF16 ? a256(R * H) : 0) + a256(R * H / 32);
      b += E * ((d.wt == MOE_BF16 ? a256(2 * I * H) + a256(H * I) : 0) + a256(2 * I * H / 32) + a256(H * I / 32));
      b += a256(R * I) + a256(R * I / 32);  // h as MXFP8
      return b;
    }
    case MOE_FP8: return mx::fp8_tensor_workspace_bytes(d, R);
  }
  return 0;
}

size_t grouped_gemm_workspace_bytes() { return a256(gemm::tail_ws_bytes(num_cus())); }

size_t mlp_bwd_workspace_bytes(const moe_mlp_desc& d, int64_t R) {
  const size_t I = d.I;
  if (d.compute == MOE_F32) return a256(4 * R * I * 4);
  if (d.compute == MOE_MXFP8) return mx::bwd_workspace_bytes(d, R);
  if (d.compute == MOE_FP8) return mx::fp8_bwd_workspace_bytes(d, R);
  return a256(R * 2 * I * 2) + a256((size_t)2 * (I / 256) * R * 4) + grouped_gemm_workspace_bytes();
}

static moe_status check_table(const void* const* t, int E, size_t align, const char* what) {
  if (!t) return fail(MOE_ERR_INVALID_ARG, std::string(what) + ": pointer table is NULL");
  for (int e = 0; e < E; ++e) {
    if (!t[e]) return fail(MOE_ERR_INVALID_ARG, std::string(what) + ": NULL pointer for expert " + std::to_string(e));
    if (!aligned(t[e], align))
      return fail(MOE_ERR_INVALID_ARG, std::string(what) + ": expert pointer not " + std::to_string(align) +
                                           "-byte aligned");
  }
  return MOE_OK;
}

static PtrTab make_tab(const void* const* t, int E) {
  PtrTab tab;
  std::memset(&tab, 0, sizeof(tab));
  for (int e = 0; e < E; ++e) tab.p[e] = t[e];
  return tab;
}

// dprob[r] = sum over j of part[j][r] in a fixed order (deterministic): 8 threads per
// row each add the partials j = q, q + 8, ... in increasing j, then the 8 sums are added
// in q order. 32 rows per workgroup, consecutive threads on consecutive rows.
__global__ __launch_bounds__(256) void reduce_partials(const float* __restrict__ part, int nparts, int64_t R,
                                                       float* __restrict__ out) {
  __shared__ float sums[8][32];
  const int rl = threadIdx.x & 31, q = threadIdx.x >> 5;
  const int64_t r = (int64_t)blockIdx.x * 32 + rl;
  float s = 0.f;
  if (r < R)
    for (int j = q; j < nparts; j += 8) s += part[(int64_t)j * R + r];
  sums[q][rl] = s;
  __syncthreads();
  if (q == 0 && r < R) {
    float t = sums[0][rl];
#pragma unroll
    for (int i = 1; i < 8; ++i) t += sums[i][rl];
    out[r] = t;
  }
}

// bf16 GroupedLinear(gate_up) + ScaledSwiGLU: h [R, I] (and z [R, 2I] when z != NULL)
// split-K tail area carved from a workspace (nullptr: the kernels never split)
struct TailArea {
  float* part = nullptr;
  int32_t* meta = nullptr;
  int cap = 0;
};
static TailArea tail_area(uint8_t* base) {
  TailArea t;
  if (!base) return t;
  t.meta = reinterpret_cast<int32_t*>(base);
  t.part = reinterpret_cast<float*>(base + gemm::kTailMetaSpace);
  t.cap = num_cus();
  return t;
}
static void set_tail(gemm::Params& p, const TailArea& t) {
  p.tail = t.part;
  p.tail_meta = t.meta;
  p.tail_cap = t.cap;
}

static moe_status bf16_gate_up(int E, int64_t R, int H, int I, const bf16_t* x, const PtrTab& w,
                               const int32_t* offsets, const float* prob, bf16_t* h, bf16_t* z, hipStream_t s,
                               const TailArea& tail = TailArea()) {
  gemm::Params p;
  std::memset(&p, 0, sizeof(p));
  set_tail(p, tail);
  std::memcpy(p.tab, w.p, sizeof(p.tab));
  p.q = x;
  p.q_ld = H;
  p.p_ld = H;
  p.c = h;
  p.c_ld = I;
  p.offsets = offsets;
  p.prob = prob;
  p.zout = z;
  p.R = R;
  p.N = 2 * I;
  p.K = H;
  p.E = E;
  p.I = I;
  p.n_tiles = I / 128;
  const int64_t mtiles = (R + gemm::kBM - 1) / gemm::kBM + E;
  return gemm::run(p, gemm::KCONTIG, gemm::KCONTIG, gemm::GROUP_M, gemm::EPI_SWIGLU, mtiles * p.n_tiles, s,
                   "grouped gate_up + ScaledSwiGLU");
}

// bf16 GroupedLinear: y [R, N] = x [R, K] W_e^T
static moe_status bf16_linear(int E, int64_t R, int K, int N, const bf16_t* x, const PtrTab& w,
                              const int32_t* offsets, bf16_t* y, hipStream_t s, const TailArea& tail = TailArea()) {
  gemm::Params q;
  std::memset(&q, 0, sizeof(q));
  set_tail(q, tail);
  std::memcpy(q.tab, w.p, sizeof(q.tab));
  q.q = x;
  q.q_ld = K;
  q.p_ld = K;
  q.c = y;
  q.c_ld = N;
  q.offsets = offsets;
  q.R = R;
  q.N = N;
  q.K = K;
  q.E = E;
  q.n_tiles = N / gemm::kBN;
  const int64_t mtiles = (R + gemm::kBM - 1) / gemm::kBM + E;
  return gemm::run(q, gemm::KCONTIG, gemm::KCONTIG, gemm::GROUP_M, gemm::EPI_STORE, mtiles * q.n_tiles, s,
                   "grouped linear");
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_grouped_mlp_fwd(const moe_mlp_desc* desc, int64_t R, const void* x_perm,
                                          const uint8_t* x_perm_scale, const void* const* w_gate_up,
                                          const void* const* w_down, const uint8_t* const* w_gate_up_scale,
                                          const uint8_t* const* w_down_scale, const int32_t* offsets,
                                          const float* prob_perm, void* y_perm, void* z_save, void* h_save,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!desc) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_mlp_fwd: desc is NULL");
  const moe_mlp_desc d = *desc;
  moe_status st = validate_desc(d, false);
  if (st != MOE_OK) return st;
  if (R < 0 || R > 0x7FFFFFFF) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_mlp_fwd: R out of [0, 2^31)");
  if (R == 0) return MOE_OK;
  const size_t align = d.compute == MOE_F32 ? 4 : 16;
  if (!x_perm || !offsets || !prob_perm || !y_perm) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_mlp_fwd: NULL pointer");
  if (!aligned(x_perm, align) || !aligned(y_perm, align))
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_mlp_fwd: x_perm / y_perm misaligned");
  if (d.save_for_bwd) {
    if (!z_save || !h_save) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_mlp_fwd: save_for_bwd needs z_save and h_save");
    if (!aligned(z_save, align) || !aligned(h_save, align))
      return fail(MOE_ERR_INVALID_ARG, "moe_grouped_mlp_fwd: z_save / h_save misaligned");
  }
  if ((st = check_table(w_gate_up, d.E, align, "moe_grouped_mlp_fwd(w_gate_up)")) != MOE_OK) return st;
  if ((st = check_table(w_down, d.E, align, "moe_grouped_mlp_fwd(w_down)")) != MOE_OK) return st;
  if (d.compute == MOE_MXFP8 && d.wt == MOE_MXFP8) {
    if ((st = check_table((const void* const*)w_gate_up_scale, d.E, 4, "moe_grouped_mlp_fwd(w_gate_up_scale)")) != MOE_OK) return st;
    if ((st = check_table((const void* const*)w_down_scale, d.E, 4, "moe_grouped_mlp_fwd(w_down_scale)")) != MOE_OK) return st;
  }
  if (d.compute == MOE_MXFP8 && d.act == MOE_MXFP8 && (!x_perm_scale || !aligned(x_perm_scale, 4)))
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_mlp_fwd: MXFP8 activations need a 4-byte aligned x_perm_scale");
  if (d.compute == MOE_FP8 && d.wt == MOE_FP8) {
    if ((st = check_table((const void* const*)w_gate_up_scale, d.E, 4, "moe_grouped_mlp_fwd(w_gate_up_scale)")) != MOE_OK) return st;
    if ((st = check_table((const void* const*)w_down_scale, d.E, 4, "moe_grouped_mlp_fwd(w_down_scale)")) != MOE_OK) return st;
  }
  if (d.compute == MOE_FP8 && d.act == MOE_FP8 && (!x_perm_scale || !aligned(x_perm_scale, 4)))
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_mlp_fwd: FP8 activations need a 4-byte aligned x_perm_scale");
  const size_t need = mlp_fwd_workspace_bytes(d, R);
  if (workspace_bytes < need) return fail(MOE_ERR_WORKSPACE, "moe_grouped_mlp_fwd: workspace too small");
  if (need > 0 && (!workspace || !aligned(workspace, 256)))
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_mlp_fwd: workspace NULL or not 256-byte aligned");
  const hipStream_t s = as_stream(stream);
  const PtrTab w1 = make_tab(w_gate_up, d.E), w2 = make_tab(w_down, d.E);

  if (d.compute == MOE_F32) {
    float* h = d.save_for_bwd ? (float*)h_save : (float*)workspace;
    return f32::forward(d, R, (const float*)x_perm, w1, w2, offsets, prob_perm, (float*)y_perm,
                        d.save_for_bwd ? (float*)z_save : nullptr, h, s);
  }
  if (d.compute == MOE_FP8) {
    return mx::forward_fp8_tensor(d, R, x_perm, reinterpret_cast<const float*>(x_perm_scale), w_gate_up, w_down,
                                  reinterpret_cast<const float* const*>(w_gate_up_scale),
                                  reinterpret_cast<const float* const*>(w_down_scale), offsets, prob_perm, y_perm,
                                  (uint8_t*)workspace, s, d.save_for_bwd ? z_save : nullptr,
                                  d.save_for_bwd ? h_save : nullptr);
  }
  if (d.compute == MOE_MXFP8) {
    return mx::forward(d, R, x_perm, x_perm_scale, w_gate_up, w_down, w_gate_up_scale, w_down_scale, offsets,
                       prob_perm, y_perm, (uint8_t*)workspace, s, d.save_for_bwd ? z_save : nullptr,
                       d.save_for_bwd ? h_save : nullptr);
  }

  // bf16: gate_up + ScaledSwiGLU (h, optionally z), then down; workspace: [h] [tail area]
  bf16_t* h = d.save_for_bwd ? (bf16_t*)h_save : (bf16_t*)workspace;
  const TailArea tail = tail_area((uint8_t*)workspace + (d.save_for_bwd ? 0 : a256((size_t)R * d.I * 2)));
  st = bf16_gate_up(d.E, R, d.H, d.I, (const bf16_t*)x_perm, w1, offsets, prob_perm, h,
                    d.save_for_bwd ? (bf16_t*)z_save : nullptr, s, tail);
  if (st != MOE_OK) return st;
  return bf16_linear(d.E, R, d.I, d.H, h, w2, offsets, (bf16_t*)y_perm, s, tail);
}

// the tail area of a caller's grouped-GEMM workspace (none if it is NULL); validated
static moe_status gemm_workspace(void* ws, size_t bytes, const char* what, TailArea* out) {
  *out = TailArea();
  if (!ws) return MOE_OK;
  if (!aligned(ws, 256)) return fail(MOE_ERR_INVALID_ARG, std::string(what) + ": workspace not 256-byte aligned");
  if (bytes < grouped_gemm_workspace_bytes()) return fail(MOE_ERR_WORKSPACE, std::string(what) + ": workspace too small");
  *out = tail_area((uint8_t*)ws);
  return MOE_OK;
}

extern "C" moe_status moe_grouped_linear(int E, int64_t R, int K, int N, moe_dtype dt, const void* x,
                                         const void* const* w, const int32_t* offsets, void* y, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_linear: E out of [1, 256]");
  if (R < 0 || R > 0x7FFFFFFF || K < 1 || N < 1) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_linear: bad R/K/N");
  if (dt != MOE_BF16 && dt != MOE_F32) return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_linear: dtype must be BF16 or F32");
  if (dt == MOE_BF16 && (N % 256 != 0 || K % 64 != 0))
    return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_linear: bf16 needs N % 256 == 0 and K % 64 == 0");
  if ((int64_t)N * K * 2 > 0x7FFFFFFFLL) return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_linear: weight exceeds 2^31 bytes");
  if (R == 0) return MOE_OK;
  const size_t align = dt == MOE_F32 ? 4 : 16;
  if (!x || !y || !offsets) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_linear: NULL pointer");
  if (!aligned(x, align) || !aligned(y, align)) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_linear: misaligned tensor");
  moe_status st = check_table(w, E, align, "moe_grouped_linear(w)");
  if (st != MOE_OK) return st;
  const PtrTab tab = make_tab(w, E);
  const hipStream_t s = as_stream(stream);
  if (dt == MOE_F32) return f32::linear(E, R, K, N, (const float*)x, tab, offsets, (float*)y, s);
  TailArea tail;
  if ((st = gemm_workspace(workspace, workspace_bytes, "moe_grouped_linear", &tail)) != MOE_OK) return st;
  return bf16_linear(E, R, K, N, (const bf16_t*)x, tab, offsets, (bf16_t*)y, s, tail);
}

extern "C" moe_status moe_grouped_gate_up_swiglu(int E, int64_t R, int H, int I, moe_dtype dt, const void* x,
                                                 const uint8_t* x_scale, const void* const* w,
                                                 const uint8_t* const* w_scale, const int32_t* offsets,
                                                 const float* prob, void* h, uint8_t* h_scale, void* z_save,
                                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gate_up_swiglu: E out of [1, 256]");
  if (R < 0 || R > 0x7FFFFFFF || H < 1 || I < 1) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gate_up_swiglu: bad R/H/I");
  if (dt != MOE_BF16 && dt != MOE_F32 && dt != MOE_MXFP8)
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gate_up_swiglu: bad dtype");
  if (dt != MOE_F32 && (H % 256 != 0 || I % 128 != 0))
    return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_gate_up_swiglu: needs H % 256 == 0 and I % 128 == 0");
  if ((int64_t)2 * I * H * 2 > 0x7FFFFFFFLL) return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_gate_up_swiglu: weight exceeds 2^31 bytes");
  if (dt == MOE_MXFP8 && z_save) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gate_up_swiglu: z_save needs BF16 or F32");
  if (R == 0) return MOE_OK;
  const size_t align = dt == MOE_F32 ? 4 : 16;
  if (!x || !h || !offsets || !prob) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gate_up_swiglu: NULL pointer");
  if (!aligned(x, align) || !aligned(h, align) || (z_save && !aligned(z_save, align)))
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gate_up_swiglu: misaligned tensor");
  moe_status st = check_table(w, E, align, "moe_grouped_gate_up_swiglu(w)");
  if (st != MOE_OK) return st;
  const hipStream_t s = as_stream(stream);
  const PtrTab tab = make_tab(w, E);
  if (dt == MOE_MXFP8) {
    if (!x_scale || !h_scale) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gate_up_swiglu: MXFP8 needs x_scale and h_scale");
    if ((st = check_table((const void* const*)w_scale, E, 4, "moe_grouped_gate_up_swiglu(w_scale)")) != MOE_OK) return st;
    return mx::gate_up(E, R, H, I, (const uint8_t*)x, x_scale, w, w_scale, offsets, prob, (uint8_t*)h, h_scale, s);
  }
  if (dt == MOE_F32)
    return f32::gate_up(E, R, H, I, (const float*)x, tab, offsets, prob, (float*)h, (float*)z_save, s);
  TailArea tail;
  if ((st = gemm_workspace(workspace, workspace_bytes, "moe_grouped_gate_up_swiglu", &tail)) != MOE_OK) return st;
  return bf16_gate_up(E, R, H, I, (const bf16_t*)x, tab, offsets, prob, (bf16_t*)h, (bf16_t*)z_save, s, tail);
}

extern "C" moe_status moe_grouped_mlp_bwd(const moe_mlp_desc* desc, int64_t R, const void* dy_perm,
                                          const void* x_perm, const void* z_save, const void* h_save,
                                          const float* prob_perm, const void* const* w_gate_up,
                                          const void* const* w_down, const int32_t* offsets, void* dx_perm,
                                          void* const* dw_gate_up, void* const* dw_down, float* dprob_perm,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!desc) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_mlp_bwd: desc is NULL");
  const moe_mlp_desc d = *desc;
  moe_status st = validate_desc(d, true);
  if (st != MOE_OK) return st;
  if (R < 0 || R > 0x7FFFFFFF) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_mlp_bwd: R out of [0, 2^31)");
  const size_t align = d.compute == MOE_F32 ? 4 : 16;
  if (!offsets) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_mlp_bwd: offsets is NULL");
  if (R > 0) {
    if (!dy_perm || !x_perm || !z_save || !h_save || !prob_perm || !dx_perm || !dprob_perm)
      return fail(MOE_ERR_INVALID_ARG, "moe_grouped_mlp_bwd: NULL pointer");
    for (const void* ptr : {dy_perm, x_perm, z_save, h_save, (const void*)dx_perm})
      if (!aligned(ptr, align)) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_mlp_bwd: misaligned tensor");
  }
  if ((st = check_table(w_gate_up, d.E, align, "moe_grouped_mlp_bwd(w_gate_up)")) != MOE_OK) return st;
  if ((st = check_table(w_down, d.E, align, "moe_grouped_mlp_bwd(w_down)")) != MOE_OK) return st;
  if ((st = check_table((const void* const*)dw_gate_up, d.E, align, "moe_grouped_mlp_bwd(dw_gate_up)")) != MOE_OK) return st;
  if ((st = check_table((const void* const*)dw_down, d.E, align, "moe_grouped_mlp_bwd(dw_down)")) != MOE_OK) return st;
  const size_t need = mlp_bwd_workspace_bytes(d, R);
  if (workspace_bytes < need) return fail(MOE_ERR_WORKSPACE, "moe_grouped_mlp_bwd: workspace too small");
  if (need > 0 && (!workspace || !aligned(workspace, 256)))
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_mlp_bwd: workspace NULL or not 256-byte aligned");
  const hipStream_t s = as_stream(stream);
  const PtrTab w1 = make_tab(w_gate_up, d.E), w2 = make_tab(w_down, d.E);
  const PtrTab dw1 = make_tab((const void* const*)dw_gate_up, d.E), dw2 = make_tab((const void* const*)dw_down, d.E);

  if (d.compute == MOE_F32) {
    return f32::backward(d, R, (const float*)dy_perm, (const float*)x_perm, (const float*)z_save,
                         (const float*)h_save, prob_perm, w1, w2, offsets, (float*)dx_perm, dw1, dw2, dprob_perm,
                         (float*)workspace, s);
  }

  if (d.compute == MOE_MXFP8) {
    return mx::backward(d, R, (const bf16_t*)dy_perm, (const bf16_t*)x_perm, (const bf16_t*)z_save,
                        (const bf16_t*)h_save, prob_perm, w_gate_up, w_down, offsets, (bf16_t*)dx_perm, dw_gate_up,
                        dw_down, dprob_perm, (uint8_t*)workspace, s);
  }
  if (d.compute == MOE_FP8) {
    return mx::backward_fp8_tensor(d, R, (const bf16_t*)dy_perm, (const bf16_t*)x_perm, (const bf16_t*)z_save,
                                   (const bf16_t*)h_save, prob_perm, w_gate_up, w_down, offsets, (bf16_t*)dx_perm,
                                   dw_gate_up, dw_down, dprob_perm, (uint8_t*)workspace, s);
  }

  const int64_t H = d.H, I = d.I;
  uint8_t* ws = (uint8_t*)workspace;
  bf16_t* dz = (bf16_t*)ws;
  ws += a256(R * 2 * I * 2);
  float* part = (float*)ws;
  ws += a256((size_t)2 * (I / 256) * R * 4);
  const TailArea tail = tail_area(ws);  // split-K tail of the gate_up dgrad
  const int64_t mtiles = (R + gemm::kBM - 1) / gemm::kBM + d.E;

  if (R > 0) {
    // down dgrad with the dSwiGLU / dprob epilogue: dH = dY W2_e (W2_e is [H][I]: K rows, I contiguous)
    gemm::Params p;
    std::memset(&p, 0, sizeof(p));
    std::memcpy(p.tab, w2.p, sizeof(p.tab));
    p.q = (const bf16_t*)dy_perm;
    p.q_ld = H;
    p.p_ld = I;
    p.c = dz;
    p.c_ld = 2 * I;
    p.offsets = offsets;
    p.prob = prob_perm;
    p.zin = (const bf16_t*)z_save;
    p.part = part;
    p.R = R;
    p.N = (int)I;
    p.K = (int)H;
    p.E = d.E;
    p.I = (int)I;
    p.n_tiles = (int)(I / gemm::kBN);
    st = gemm::run(p, gemm::MNCONTIG, gemm::KCONTIG, gemm::GROUP_M, gemm::EPI_DSWIGLU, mtiles * p.n_tiles, s,
                   "moe_grouped_mlp_bwd(down dgrad)");
    if (st != MOE_OK) return st;
    hipLaunchKernelGGL(reduce_partials, dim3((unsigned)((R + 31) / 32)), dim3(256), 0, s, (const float*)part,
                       2 * p.n_tiles, R, dprob_perm);
    if ((st = check_launch("moe_grouped_mlp_bwd(dprob)")) != MOE_OK) return st;

    // gate_up dgrad: dX = dZ W1_e (W1_e is [2I][H]: K rows, H contiguous)
    gemm::Params q;
    std::memset(&q, 0, sizeof(q));
    std::memcpy(q.tab, w1.p, sizeof(q.tab));
    q.q = dz;
    q.q_ld = 2 * I;
    q.p_ld = H;
    q.c = (bf16_t*)dx_perm;
    q.c_ld = H;
    q.offsets = offsets;
    q.R = R;
    q.N = (int)H;
    q.K = (int)(2 * I);
    q.E = d.E;
    q.I = (int)I;
    q.n_tiles = (int)(H / gemm::kBN);
    set_tail(q, tail);
    st = gemm::run(q, gemm::MNCONTIG, gemm::KCONTIG, gemm::GROUP_M, gemm::EPI_STORE, mtiles * q.n_tiles, s,
                   "moe_grouped_mlp_bwd(gate_up dgrad)");
    if (st != MOE_OK) return st;
  }

  // down wgrad: dW2_e[h][i] = sum_r dY[r][h] * Hs[r][i]
  gemm::Params w;
  std::memset(&w, 0, sizeof(w));
  std::memcpy(w.tab, dw2.p, sizeof(w.tab));
  w.p = (const bf16_t*)h_save;
  w.p_ld = I;
  w.q = (const bf16_t*)dy_perm;
  w.q_ld = H;
  w.c_ld = I;
  w.offsets = offsets;
  w.R = R;
  w.M = (int)H;
  w.N = (int)I;
  w.E = d.E;
  w.I = (int)I;
  w.n_tiles = (int)(I / gemm::kBN);
  st = gemm::run(w, gemm::MNCONTIG, gemm::MNCONTIG, gemm::GROUP_K, gemm::EPI_STORE,
                 (int64_t)d.E * (H / gemm::kBM) * w.n_tiles, s, "moe_grouped_mlp_bwd(down wgrad)");
  if (st != MOE_OK) return st;

  // gate_up wgrad: dW1_e[j][h] = sum_r dZ[r][j] * X[r][h]
  gemm::Params v;
  std::memset(&v, 0, sizeof(v));
  std::memcpy(v.tab, dw1.p, sizeof(v.tab));
  v.p = (const bf16_t*)x_perm;
  v.p_ld = H;
  v.q = dz;
  v.q_ld = 2 * I;
  v.c_ld = H;
  v.offsets = offsets;
  v.R = R;
  v.M = (int)(2 * I);
  v.N = (int)H;
  v.E = d.E;
  v.I = (int)I;
  v.n_tiles = (int)(H / gemm::kBN);
  return gemm::run(v, gemm::MNCONTIG, gemm::MNCONTIG, gemm::GROUP_K, gemm::EPI_STORE,
                   (int64_t)d.E * (2 * I / gemm::kBM) * v.n_tiles, s, "moe_grouped_mlp_bwd(gate_up wgrad)");
}
