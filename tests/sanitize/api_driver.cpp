// Drives the host side of the C ABI -- descriptor validation, plans, the
// tile schedule, workspace sizing and the run-time argument checks that
// precede any device call -- for a build with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py).  The kernel
// launchers are replaced by stubs: no device code is involved.  Exit status
// 0 when every status matches what the header promises.
#include <cstdio>
#include <cstring>
#include <vector>

#include "kernels.h"
#include "swa_sdpa.h"

namespace swa {
hipError_t launch_bwd_dot(const BwdArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_clear(const BwdArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_main(const BwdArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_dq(const BwdArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_stream(const BwdArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_dsink(const BwdArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_fwd(const FwdArgs&, hipStream_t) { return hipSuccess; }
}  // namespace swa

static int failures = 0;
static void expect(bool ok, const char* what) {
  if (!ok) {
    std::printf("FAILED: %s (%s)\n", what, sdpa_last_error());
    ++failures;
  }
}

static sdpa_attn_desc desc(int B, int Hq, int Hkv, int D, int Sq, int Skv) {
  sdpa_attn_desc d;
  std::memset(&d, 0, sizeof d);
  d.dtype = SDPA_BF16;
  d.layout = SDPA_LAYOUT_BHSD;
  d.batch = B;
  d.heads_q = Hq;
  d.heads_kv = Hkv;
  d.head_dim = D;
  d.seq_q = Sq;
  d.seq_kv = Skv;
  d.causal = 1;
  d.window_left = 64;
  d.scale = 0.125f;
  auto set = [&](int64_t* st, int H, int S) {
    st[0] = (int64_t)H * S * D;
    st[1] = (int64_t)S * D;
    st[2] = D;
  };
  for (int64_t* st : {d.stride_q, d.stride_o, d.stride_do, d.stride_dq}) set(st, Hq, Sq);
  for (int64_t* st : {d.stride_k, d.stride_v, d.stride_dk, d.stride_dv}) set(st, Hkv, Skv);
  return d;
}

int main() {
  // valid plans over the kernel choices, in all three dQ modes
  struct Case {
    int B, Hq, Hkv, D, Sq, Skv, W, R, br, causal;
  } cases[] = {{2, 4, 4, 64, 1000, 1000, 128, 0, 0, 1},  {2, 8, 2, 128, 200, 333, 100, 70, 1, 1},
               {1, 4, 1, 64, 190, 190, -1, 0, 0, 1},     {1, 2, 2, 64, 100, 250, 50, 0, 1, 0},
               {1, 2, 2, 128, 0, 0, 5, 0, 0, 1},         {3, 6, 3, 64, 64, 4096, 2047, 9, 1, 1}};
  for (const Case& c : cases)
    for (int det = 0; det <= 2; ++det) {
      sdpa_attn_desc d = desc(c.B, c.Hq, c.Hkv, c.D, c.Sq, c.Skv);
      d.window_left = c.W;
      d.window_right = c.R;
      d.bottom_right = c.br;
      d.causal = c.causal;
      d.deterministic = det;
      sdpa_bwd_plan_t* plan = nullptr;
      size_t ws = 0;
      expect(sdpa_bwd_plan(&d, &plan, &ws) == SDPA_OK && plan && ws % 256 == 0, "valid backward plan");
      if (!plan) continue;
      // the schedule over several lengths, into exactly sized arrays
      for (int lq : {0, 1, 63, 64, 65, 777})
        for (int lk : {0, 1, 128, 129, 4096}) {
          int32_t tq, tk, nq, nk;
          expect(sdpa_bwd_schedule(plan, lq, lk, &tq, &tk, &nq, &nk, 0, nullptr, nullptr, 0, nullptr, nullptr) ==
                     SDPA_OK,
                 "schedule size query");
          std::vector<int32_t> qlo(nk > 0 ? nk : 1), qhi(nk > 0 ? nk : 1), kf(nq > 0 ? nq : 1), kl(nq > 0 ? nq : 1);
          expect(sdpa_bwd_schedule(plan, lq, lk, &tq, &tk, &nq, &nk, nk, qlo.data(), qhi.data(), nq, kf.data(),
                                   kl.data()) == SDPA_OK,
                 "schedule");
        }
      // run-time checks that precede any device call
      sdpa_bwd_tensors t;
      std::memset(&t, 0, sizeof t);
      if (ws) expect(sdpa_bwd_run(plan, &t, nullptr, ws - 1, nullptr) == SDPA_ERR_WORKSPACE, "undersized workspace");
      expect(sdpa_bwd_run(plan, nullptr, nullptr, ws, nullptr) == SDPA_ERR_INVALID_ARG, "null tensors");
      sdpa_bwd_plan_destroy(plan);
      sdpa_fwd_plan_t* fplan = nullptr;
      expect(sdpa_fwd_plan(&d, &fplan, &ws) == SDPA_OK && fplan, "valid forward plan");
      sdpa_fwd_plan_destroy(fplan);
    }
  // invalid descriptors are rejected with a message naming the field
  struct Bad {
    const char* field;
    void (*edit)(sdpa_attn_desc&);
    sdpa_status want;
  } bad[] = {{"head_dim", [](sdpa_attn_desc& d) { d.head_dim = 96; }, SDPA_ERR_UNSUPPORTED},
             {"heads_q", [](sdpa_attn_desc& d) { d.heads_q = 5; }, SDPA_ERR_INVALID_ARG},
             {"window_left", [](sdpa_attn_desc& d) { d.window_left = -7; }, SDPA_ERR_INVALID_ARG},
             {"window_right", [](sdpa_attn_desc& d) { d.window_right = -1; }, SDPA_ERR_INVALID_ARG},
             {"deterministic", [](sdpa_attn_desc& d) { d.deterministic = 3; }, SDPA_ERR_INVALID_ARG},
             {"q_run_tiles", [](sdpa_attn_desc& d) { d.q_run_tiles = 17; }, SDPA_ERR_INVALID_ARG},
             {"stride_q", [](sdpa_attn_desc& d) { d.stride_q[2] = 60; }, SDPA_ERR_INVALID_ARG},
             {"scale", [](sdpa_attn_desc& d) { d.scale = 0.f; }, SDPA_ERR_INVALID_ARG}};
  for (const Bad& b : bad) {
    sdpa_attn_desc d = desc(2, 4, 2, 64, 300, 300);
    b.edit(d);
    sdpa_bwd_plan_t* plan = nullptr;
    size_t ws = 0;
    const sdpa_status st = sdpa_bwd_plan(&d, &plan, &ws);
    expect(st == b.want && !plan && std::strstr(sdpa_last_error(), b.field), b.field);
  }
  expect(sdpa_bwd_plan(nullptr, nullptr, nullptr) == SDPA_ERR_INVALID_ARG, "null out-pointers");
  expect(std::strcmp(sdpa_status_string(SDPA_ERR_WORKSPACE), "SDPA_ERR_WORKSPACE") == 0, "status string");
  std::printf("%s\n", failures ? "api driver: FAILED" : "api driver: ok");
  return failures ? 1 : 0;
}
