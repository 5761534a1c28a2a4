// Host-side argument checks of every entry point in include/moe.h, built
// with AddressSanitizer on the host code only (tests/test_host_asan.py):
// each call below must be rejected before anything is enqueued, and the
// size queries must answer without touching a device.  Stand-in pointers
// are never dereferenced by a call that rejects its arguments; a read or
// write through one, or any other host memory error on these paths, is an
// AddressSanitizer report and a failed run.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "moe.h"

namespace {

int failures = 0;

void expect(const char* what, int got, int want) {
  if (got != want) {
    std::printf("FAIL %s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

// a non-null stand-in for a device pointer: outside any host allocation
void* const P = reinterpret_cast<void*>(uintptr_t(4096));
template <typename T>
T* p() { return static_cast<T*>(P); }

}  // namespace

int main() {
  // route
  expect("route x=NULL", moe_route(nullptr, MOE_BF16, 64, 64, p<float>(), nullptr, nullptr, 8, 2, 0,
                                   p<int32_t>(), p<float>(), p<float>(), nullptr), MOE_EINVAL);
  expect("route k>E", moe_route(P, MOE_BF16, 64, 64, p<float>(), nullptr, nullptr, 8, 9, 0,
                                p<int32_t>(), p<float>(), p<float>(), nullptr), MOE_EINVAL);
  expect("route E too large", moe_route(P, MOE_BF16, 64, 64, p<float>(), nullptr, nullptr, 1025, 2, 0,
                                        p<int32_t>(), p<float>(), p<float>(), nullptr), MOE_ENOTSUP);
  expect("route d", moe_route(P, MOE_BF16, 64, 60, p<float>(), nullptr, nullptr, 8, 2, 0,
                              p<int32_t>(), p<float>(), p<float>(), nullptr), MOE_ENOTSUP);
  expect("replay idx=NULL", moe_route_replay(P, MOE_BF16, 64, 64, p<float>(), nullptr, 8, 2, 0, nullptr,
                                             p<float>(), p<float>(), nullptr), MOE_EINVAL);
  expect("replay uniform", moe_route_replay(P, MOE_BF16, 64, 64, p<float>(), nullptr, 8, 2, MOE_UNIFORM_GATES,
                                            p<int32_t>(), p<float>(), p<float>(), nullptr), MOE_EINVAL);
  expect("hash ids=NULL", moe_route_hash(nullptr, 64, 8, 2, 0, p<int32_t>(), p<float>(), nullptr), MOE_EINVAL);
  expect("hash k", moe_route_hash(p<int32_t>(), 64, 64, 17, 0, p<int32_t>(), p<float>(), nullptr), MOE_ENOTSUP);

  // permute family
  const size_t pw = moe_workspace_size(MOE_CALL_PERMUTE, 1000, 8, 64, 64, 0);
  expect("permute no workspace", moe_permute(p<int32_t>(), 1000, 8, 64, P, MOE_BF16, 64, p<int32_t>(),
                                             p<int32_t>(), p<int32_t>(), p<int32_t>(), P, nullptr, pw, nullptr),
         MOE_EWORKSPACE);
  expect("permute small workspace", moe_permute(p<int32_t>(), 1000, 8, 64, P, MOE_BF16, 64, p<int32_t>(),
                                                p<int32_t>(), p<int32_t>(), p<int32_t>(), P, P, pw - 1, nullptr),
         MOE_EWORKSPACE);
  expect("permute copy without x", moe_permute(p<int32_t>(), 1000, 8, 64, nullptr, MOE_BF16, 64, p<int32_t>(),
                                               p<int32_t>(), p<int32_t>(), p<int32_t>(), P, P, pw, nullptr),
         MOE_EINVAL);
  expect("permute rows", moe_permute(p<int32_t>(), 1000, 8, 64, P, MOE_BF16, 4, p<int32_t>(), p<int32_t>(),
                                     p<int32_t>(), p<int32_t>(), P, P, pw, nullptr), MOE_ENOTSUP);
  expect("permute_capacity row_of=NULL",
         moe_permute_capacity(p<int32_t>(), 1000, 8, 64, 200, P, MOE_BF16, 64, p<int32_t>(), p<int32_t>(), nullptr,
                              p<int32_t>(), P, P, pw, nullptr), MOE_EINVAL);
  expect("permute_noalloc counts=NULL",
         moe_permute_noalloc(p<int32_t>(), 1000, 8, 64, P, MOE_BF16, 64, nullptr, p<int32_t>(), p<int32_t>(),
                             p<int32_t>(), P, nullptr), MOE_EINVAL);
  expect("permute_noalloc histogram past the scratch",
         moe_permute_noalloc(p<int32_t>(), 1 << 20, 8, 1024, nullptr, MOE_BF16, 64, p<int32_t>(), p<int32_t>(),
                             p<int32_t>(), p<int32_t>(), nullptr, nullptr), MOE_ENOTSUP);

  // grouped FFN family
  const size_t fw = moe_workspace_size(MOE_CALL_GROUPED_FFN, 1000, 1, 64, 256, 128);
  expect("ffn h=NULL", moe_grouped_ffn(P, 1000, 256, MOE_BF16, p<int32_t>(), 64, 128, P, P, nullptr, nullptr,
                                       p<float>(), P, fw, nullptr), MOE_EINVAL);
  expect("ffn d", moe_grouped_ffn(P, 1000, 96, MOE_BF16, p<int32_t>(), 64, 128, P, P, nullptr, P, p<float>(), P,
                                  fw, nullptr), MOE_ENOTSUP);
  expect("ffn workspace", moe_grouped_ffn(P, 1000, 256, MOE_BF16, p<int32_t>(), 64, 128, P, P, nullptr, P,
                                          p<float>(), P, 0, nullptr), MOE_EWORKSPACE);
  expect("ffn_gather token_of=NULL",
         moe_grouped_ffn_gather(P, 256, nullptr, 512, 128, MOE_BF16, p<int32_t>(), 4, 128, P, P, nullptr, P,
                                p<float>(), P, fw, nullptr), MOE_EINVAL);
  expect("pack f", moe_pack_expert_weights(P, P, 4, 256, 192, P, P, nullptr), MOE_ENOTSUP);
  expect("pack NULL", moe_pack_expert_weights(nullptr, P, 4, 256, 256, P, P, nullptr), MOE_EINVAL);
  expect("ffn_packed f", moe_grouped_ffn_packed(P, 1000, p<int32_t>(), 1000, 256, p<int32_t>(), 64, 192, P, P,
                                                nullptr, P, p<float>(), P, fw, nullptr), MOE_ENOTSUP);
  expect("ffn_packed workspace", moe_grouped_ffn_packed(P, 1000, p<int32_t>(), 1000, 256, p<int32_t>(), 64, 256, P,
                                                        P, nullptr, P, p<float>(), P, 0, nullptr), MOE_EWORKSPACE);
  if (moe_packed_weight_bytes(1, 3, 192, 256) != size_t(3) * 256 * 256 * 2 || moe_packed_weight_bytes(7, 3, 192, 256))
    std::printf("FAIL packed weight bytes\n"), ++failures;
  {
    void* ev[MOE_FFN_STAGES] = {P, P};   // taken by the next grouped FFN call, which fails its checks first
    expect("ffn stage events", moe_ffn_stage_events(ev), MOE_OK);
    expect("ffn h=NULL after events", moe_grouped_ffn(P, 1000, 256, MOE_BF16, p<int32_t>(), 64, 128, P, P, nullptr,
                                                      nullptr, p<float>(), P, fw, nullptr), MOE_EINVAL);
    expect("ffn stage events cleared", moe_ffn_stage_events(nullptr), MOE_OK);
  }

  // combine, bias update, aux loss
  expect("combine y=NULL", moe_combine(nullptr, p<int32_t>(), p<float>(), nullptr, 10, 2, 64, P, MOE_F32, nullptr),
         MOE_EINVAL);
  expect("combine d", moe_combine(p<float>(), p<int32_t>(), p<float>(), nullptr, 10, 2, 66, P, MOE_F32, nullptr),
         MOE_ENOTSUP);
  expect("bias k>E", moe_bias_update(p<float>(), p<int32_t>(), 8, 64, 9, 1e-3f, nullptr), MOE_EINVAL);
  const size_t aw = moe_workspace_size(MOE_CALL_AUX_LOSS, 1000, 8, 64, 0, 0);
  expect("aux uniform", moe_aux_loss(p<float>(), p<int32_t>(), 1000, 64, 8, MOE_UNIFORM_GATES, 0.01f, p<float>(),
                                     nullptr, P, aw, nullptr), MOE_EINVAL);
  expect("aux workspace", moe_aux_loss(p<float>(), p<int32_t>(), 1000, 64, 8, MOE_SIGMOID_NORM, 0.01f, p<float>(),
                                       nullptr, P, aw - 1, nullptr), MOE_EWORKSPACE);

  // backward: a full argument block, then one fault at a time
  moe_bwd_args a;
  std::memset(&a, 0, sizeof(a));
  a.struct_size = sizeof(a);
  a.T = 1000, a.d = 256, a.f = 128, a.E = 64, a.k = 8, a.score_fn = MOE_SQRT_SOFTPLUS_NORM;
  a.dy = a.x = P;
  a.w_router = a.logits = p<float>();
  a.topk_idx = a.row_of = a.token_of = a.offsets = p<int32_t>();
  a.topk_gate = p<float>();
  a.gu_saved = a.h = a.w_gate_up = a.w_down = P;
  a.dx = a.dw_router = a.dw_gate_up = a.dw_down = p<float>();
  a.workspace = P;
  a.workspace_bytes = moe_workspace_size(MOE_CALL_BACKWARD, a.T, a.k, a.E, a.d, a.f);
  moe_bwd_args b = a;
  b.struct_size = 8;
  expect("backward struct_size", moe_backward(&b, nullptr), MOE_EINVAL);
  b = a, b.dy = nullptr;
  expect("backward dy=NULL", moe_backward(&b, nullptr), MOE_EINVAL);
  b = a, b.k = 65;
  expect("backward k", moe_backward(&b, nullptr), MOE_EINVAL);
  b = a, b.workspace_bytes -= 1;
  expect("backward workspace", moe_backward(&b, nullptr), MOE_EWORKSPACE);
  b = a, b.d = 96;
  expect("backward d", moe_backward(&b, nullptr), MOE_ENOTSUP);
  b = a, b.aux_alpha = 0.5f;   // the aux loss needs counts
  expect("backward aux without counts", moe_backward(&b, nullptr), MOE_EINVAL);
  b = a, b.f_shared = 128, b.w_gate_up_shared = b.w_down_shared = b.gu_shared = b.h_shared = P;
  b.dw_gate_up_shared = b.dw_down_shared = p<float>();
  b.workspace_shared = P, b.workspace_shared_bytes = 0;
  expect("backward shared workspace", moe_backward(&b, nullptr), MOE_EWORKSPACE);

  // size queries over a grid of shapes, and every status string
  size_t acc = 0;
  for (int which = 0; which <= 6; ++which)
    for (int64_t T : {1, 7, 1000, 16384})
      for (int k : {1, 2, 8})
        for (int E : {1, 8, 64, 256})
          for (int64_t d : {64, 2048, 7168})
            for (int64_t f : {64, 1024, 14336}) acc += moe_workspace_size(which, T, k, E, d, f) & 1;
  for (int s = -1; s <= 6; ++s) {
    const char* m = moe_status_str(static_cast<moe_status>(s));
    if (!m || !std::strlen(m)) std::printf("FAIL status string %d\n", s), ++failures;
  }
  std::printf("%s: %d failed checks (%zu odd sizes)\n", failures ? "FAIL" : "ok", failures, acc);
  return failures ? 1 : 0;
}
