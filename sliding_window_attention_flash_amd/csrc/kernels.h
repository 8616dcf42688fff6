// Kernel launch interface between the C-ABI layer (api.cpp) and the HIP
// kernels (bwd.hip, fwd.hip).  Internal; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace swa {

struct BwdArgs {
  Problem p;
  int dtype;  // 0 bf16, 1 f16
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const float* lse;
  const float* sink;
  void* dq;
  void* dk;
  void* dv;
  float* dsink;
  // workspace
  float* delta;      // [stat rows]
  float* dq_acc;     // [stat rows, D] fp32 dQ accumulator / relay partials
  float* dq_stash;   // [stat rows, D] streaming relay: partials awaiting their turn
  int* sem;          // [B, Hq, n_q_tiles] relay turn counters
  int* ctl;          // [0] tile ticket, [1] relay watchdog expiries
  float* sink_part;  // [Hq, B, n_q_tiles] per-q-tile dSink partials
  int deterministic;
  int spin_limit;    // relay watchdog: spins before a wait gives up
  int relay_bias;    // added to every relay wait's target turn: 0, or (test
                     // hook) a turn no visitor ever releases
};

struct FwdArgs {
  Problem p;
  int dtype;
  const void* q;
  const void* k;
  const void* v;
  const float* sink;
  void* o;
  float* lse;
};

hipError_t launch_bwd_dot(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_clear(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_main(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_stream(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_qstream(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dsink(const BwdArgs& a, hipStream_t stream);
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);

}  // namespace swa
