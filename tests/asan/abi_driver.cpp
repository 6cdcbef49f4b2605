// Host-side check of the C-ABI under AddressSanitizer: linked with the library's
// objects compiled with -fsanitize=address for the host, it calls every entry point on
// paths that end before any launch (argument, size, alignment and workspace checks,
// workspace-size queries, status strings) and checks each status. Any heap or stack
// error in that host code (the checks, the error-message strings, the descriptor
// and table handling) is reported by the sanitizer and fails the run. It also checks
// the grouped GEMMs' tile order inside an expert, compiled for the host.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "gemm_common.h"
#include "moe.h"

static int g_failures = 0;

static void expect(const char* what, moe_status got, moe_status want) {
  const char* msg = moe_last_error();
  const size_t len = msg ? std::strlen(msg) : 0;  // the sanitizer checks this read
  if (got != want || (want != MOE_OK && len == 0)) {
    std::printf("FAIL %s: status %d (%s), expected %d; last error '%s'\n", what, (int)got, moe_status_str(got),
                (int)want, msg ? msg : "(null)");
    ++g_failures;
  }
}

int main() {
  const moe_status OK = MOE_OK, INV = MOE_ERR_INVALID_ARG, UNS = MOE_ERR_UNSUPPORTED, WS = MOE_ERR_WORKSPACE;
  // status strings, including values outside the enum
  for (int s = -3; s < 12; ++s) {
    const char* t = moe_status_str((moe_status)s);
    if (!t || std::strlen(t) == 0) {
      std::printf("FAIL moe_status_str(%d)\n", s);
      ++g_failures;
    }
  }

  // routing
  expect("route E=0", moe_route_topk(nullptr, 10, 0, 1, 1, nullptr, nullptr, nullptr), INV);
  expect("route k>E", moe_route_topk(nullptr, 10, 8, 9, 1, nullptr, nullptr, nullptr), INV);
  expect("route k>16", moe_route_topk(nullptr, 10, 32, 17, 1, nullptr, nullptr, nullptr), UNS);
  expect("route T=0", moe_route_topk(nullptr, 0, 8, 2, 1, nullptr, nullptr, nullptr), OK);
  expect("route NULL", moe_route_topk(nullptr, 5, 8, 2, 1, nullptr, nullptr, nullptr), INV);
  expect("router logits NULL", moe_router_logits(nullptr, nullptr, 4, 256, 8, nullptr, nullptr), INV);
  expect("route bwd NULL",
         moe_route_topk_bwd(nullptr, nullptr, nullptr, nullptr, 4, 8, 2, 1, nullptr, nullptr), INV);
  expect("router bwd NULL",
         moe_router_bwd(nullptr, nullptr, nullptr, nullptr, 4, 256, 8, nullptr, nullptr, nullptr, 0, nullptr), INV);

  // permutation and combine
  expect("permute NULL", moe_permute(nullptr, nullptr, MOE_BF16, 4, 256, 8, 2, nullptr, nullptr, 0, nullptr, nullptr,
                                     nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr), INV);
  expect("permute k>E", moe_permute(nullptr, nullptr, MOE_BF16, 4, 256, 2, 3, nullptr, nullptr, 0, nullptr, nullptr,
                                    nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr), INV);
  expect("permute noalloc past its scratch",
         moe_permute_noalloc(nullptr, nullptr, MOE_BF16, (int64_t)1 << 40, 256, 8, 2, nullptr, nullptr, 0, nullptr,
                             nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), UNS);
  expect("combine MXFP8", moe_unpermute_combine(nullptr, MOE_MXFP8, nullptr, nullptr, 4, 8, 2, nullptr, nullptr), UNS);
  expect("combine grid", moe_unpermute_combine(nullptr, MOE_BF16, nullptr, nullptr, (int64_t)1 << 34, 8, 2, nullptr,
                                               nullptr), UNS);
  expect("combine NULL", moe_unpermute_combine(nullptr, MOE_BF16, nullptr, nullptr, 4, 8, 2, nullptr, nullptr), INV);

  // quantisers
  expect("mxfp8 cols%32", mxfp8_quantize(nullptr, 4, 33, nullptr, nullptr, nullptr), INV);
  expect("mxfp8 NULL", mxfp8_quantize(nullptr, 4, 64, nullptr, nullptr, nullptr), INV);
  expect("mxfp8 colwise NULL",
         mxfp8_quantize_colwise(nullptr, 256, 64, 2, nullptr, 32, 256, nullptr, nullptr, nullptr, nullptr), INV);
  expect("mxfp8 pack rows", mxfp8_pack_weight_bwd(nullptr, 100, 64, nullptr, nullptr), UNS);
  expect("fp8 NULL", fp8_tensor_quantize(nullptr, 64, nullptr, nullptr, nullptr), INV);
  expect("fp8 colwise NULL",
         fp8_tensor_quantize_colwise(nullptr, 256, 64, 2, nullptr, 32, 256, nullptr, nullptr, nullptr, nullptr), INV);
  expect("fp8 pack NULL", fp8_tensor_pack_weight_bwd(nullptr, 128, 64, nullptr, nullptr), INV);
  expect("mx weights n=0", mxfp8_quantize_weights(0, nullptr, 128, 64, nullptr, nullptr, nullptr, nullptr), INV);
  expect("mx weights NULL table", mxfp8_quantize_weights(2, nullptr, 128, 64, nullptr, nullptr, nullptr, nullptr), INV);
  {
    const void* w[2] = {nullptr, nullptr};
    uint8_t* c[2] = {nullptr, nullptr};
    void* p[2] = {nullptr, nullptr};
    expect("mx weights NULL entries", mxfp8_quantize_weights(2, w, 128, 64, c, c, p, nullptr), INV);
    expect("fp8 weights NULL entries", fp8_tensor_quantize_weights(2, w, 128, 64, c, nullptr, p, nullptr), INV);
  }

  // grouped GEMMs and the MLP
  moe_mlp_desc d{};
  d.E = 8; d.H = 256; d.I = 256; d.compute = MOE_BF16; d.act = MOE_BF16; d.wt = MOE_BF16; d.save_for_bwd = 1;
  expect("mlp fwd NULL desc", moe_grouped_mlp_fwd(nullptr, 4, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                                  nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr), INV);
  expect("mlp fwd NULL tensors", moe_grouped_mlp_fwd(&d, 4, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                                     nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
         INV);
  moe_mlp_desc odd = d;
  odd.H = 100;
  expect("mlp fwd bf16 H%256", moe_grouped_mlp_fwd(&odd, 4, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                                   nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
         UNS);
  moe_mlp_desc bad = d;
  bad.E = 0;
  expect("mlp bwd E=0", moe_grouped_mlp_bwd(&bad, 4, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                            nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr), INV);
  expect("mlp bwd NULL tensors", moe_grouped_mlp_bwd(&d, 4, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                                     nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                                                     nullptr), INV);
  expect("linear E=0", moe_grouped_linear(0, 4, 64, 256, MOE_BF16, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                                          nullptr), INV);
  expect("linear bf16 N%256", moe_grouped_linear(2, 4, 64, 100, MOE_BF16, nullptr, nullptr, nullptr, nullptr,
                                                 nullptr, 0, nullptr), UNS);
  expect("linear NULL", moe_grouped_linear(2, 4, 64, 256, MOE_BF16, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                                           nullptr), INV);
  expect("gate_up bad dtype", moe_grouped_gate_up_swiglu(2, 4, 256, 128, MOE_FP8, nullptr, nullptr, nullptr, nullptr,
                                                         nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                                                         nullptr), INV);
  expect("gate_up NULL", moe_grouped_gate_up_swiglu(2, 4, 256, 128, MOE_BF16, nullptr, nullptr, nullptr, nullptr,
                                                    nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
         INV);
  {
    // a table whose second entry is NULL: the table check reads exactly E entries
    alignas(256) static uint16_t buf[512];
    const void* tab[2] = {buf, nullptr};
    expect("linear NULL table entry", moe_grouped_linear(2, 4, 64, 256, MOE_BF16, buf, tab, (const int32_t*)buf, buf,
                                                         nullptr, 0, nullptr), INV);
  }

  {
    // float32 sizes whose launch grid would not fit: refused before any launch
    alignas(256) static float f[64];
    const void* tab[1] = {f};
    expect("linear f32 grid", moe_grouped_linear(1, 4, 1, 65535 * 64 + 1, MOE_F32, f, tab, (const int32_t*)f, f,
                                                 nullptr, 0, nullptr), UNS);
  }

  // workspace sizes (pure host arithmetic) and a workspace that is too small
  size_t bytes = 0;
  expect("ws NULL out", moe_workspace_size(MOE_OP_PERMUTE, nullptr, 0, 16, 8, 2, nullptr), INV);
  expect("ws permute", moe_workspace_size(MOE_OP_PERMUTE, nullptr, 0, 4096, 8, 2, &bytes), OK);
  expect("ws mlp fwd", moe_workspace_size(MOE_OP_MLP_FWD, &d, 8192, 0, 0, 0, &bytes), OK);
  expect("ws mlp bwd", moe_workspace_size(MOE_OP_MLP_BWD, &d, 8192, 0, 0, 0, &bytes), OK);
  expect("ws mlp bwd R=4", moe_workspace_size(MOE_OP_MLP_BWD, &d, 4, 0, 0, 0, &bytes), OK);
  const size_t bwd_bytes = bytes;  // what the undersized call below is measured against
  expect("ws grouped gemm", moe_workspace_size(MOE_OP_GROUPED_GEMM, nullptr, 0, 0, 1, 1, &bytes), OK);
  expect("ws router bwd", moe_workspace_size(MOE_OP_ROUTER_BWD, &d, 0, 4096, 8, 0, &bytes), OK);
  expect("ws router bwd NULL desc", moe_workspace_size(MOE_OP_ROUTER_BWD, nullptr, 0, 4096, 8, 0, &bytes), INV);
  expect("ws bad op", moe_workspace_size((moe_op)99, &d, 8192, 0, 0, 0, &bytes), INV);
  for (moe_dtype c : {MOE_F32, MOE_BF16, MOE_MXFP8, MOE_FP8}) {
    moe_mlp_desc x = d;
    x.compute = c;
    x.act = c == MOE_F32 ? MOE_F32 : MOE_BF16;
    x.wt = x.act;
    moe_workspace_size(MOE_OP_MLP_FWD, &x, 1000, 0, 0, 0, &bytes);
    moe_workspace_size(MOE_OP_MLP_BWD, &x, 1000, 0, 0, 0, &bytes);
  }
  if (bwd_bytes > 0) {
    alignas(256) static uint16_t t[2048];
    const void* tab[8];
    void* otab[8];
    for (int e = 0; e < 8; ++e) {
      tab[e] = t;
      otab[e] = t;
    }
    expect("mlp bwd workspace too small",
           moe_grouped_mlp_bwd(&d, 4, t, t, t, t, (const float*)t, tab, tab, (const int32_t*)t, t, otab, otab,
                               (float*)t, t, bwd_bytes / 2, nullptr), WS);
  }

  // The grouped GEMMs' tile order inside an expert (the only data-dependent index
  // arithmetic of their tile decode): for every expert of 1..96 row tiles and 1..64
  // column tiles it must map [0, mte * ntiles) one to one onto the tiles, in range.
  {
    std::vector<unsigned char> seen;
    int bad = 0;
    for (int mte = 1; mte <= 96 && !bad; ++mte)
      for (int nt_all = 1; nt_all <= 64 && !bad; ++nt_all) {
        seen.assign((size_t)mte * nt_all, 0);
        for (int local = 0; local < mte * nt_all; ++local) {
          int mt = -1, nt = -1;
          moe::gemm::tile_in_expert(local, mte, nt_all, mt, nt);
          if (mt < 0 || mt >= mte || nt < 0 || nt >= nt_all || seen[(size_t)mt * nt_all + nt]++) {
            std::printf("FAIL tile_in_expert(%d, %d, %d) -> (%d, %d)\n", local, mte, nt_all, mt, nt);
            bad = 1;
            break;
          }
        }
      }
    g_failures += bad;
  }

  std::printf("%s: %d failure(s)\n", g_failures ? "FAILED" : "ok", g_failures);
  return g_failures ? 1 : 0;
}
