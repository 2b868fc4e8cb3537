// Internal launch interfaces between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sr_replay.h"

namespace sr {

// Validated arguments of one gated-delta-rule replay launch.
struct GdnArgs {
  int n_seqs, total_tokens, h_k, h_v, d_k, d_v;
  int dtype_qkv, dtype_o;
  int erase, alpha_is_log;
  float scale;
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const int32_t* cu;
  const float* s0;
  float* s_out;
  void* o;
};

bool gdn_serial_supports(int d_k, int d_v);
hipError_t launch_gdn_serial(const GdnArgs& a, hipStream_t s);

bool gdn_chunk_supports(int dtype_qkv, int d_k, int d_v);
hipError_t launch_gdn_chunk(const GdnArgs& a, hipStream_t s);

}  // namespace sr
