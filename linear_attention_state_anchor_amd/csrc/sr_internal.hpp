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

// Host-side validation of the replay arguments shared by the entry points
// (SR_OK or an SR_E* status); nothing is enqueued.
int validate_gdn(const sr_gdn_desc* d, const sr_gdn_io* io, GdnArgs* out);

// Checks of device-side preconditions (validate.hip).  Each runs a kernel on
// `s`, waits for it, and returns SR_OK, SR_EDATA or an argument status.
bool debug_checks_enabled();  // SR_DEBUG=1 in the environment
int check_cu_seqlens(const int32_t* cu, int n_seqs, int total_tokens, hipStream_t s);
int check_replay(const GdnArgs& a, hipStream_t s);
int check_gather(int64_t n_blocks, int anchors_per_page, const int32_t* offsets,
                 const int32_t* pt, int pt_stride, const int32_t* m_len,
                 const int32_t* k_len, int n_req, int total, hipStream_t s);

}  // namespace sr
