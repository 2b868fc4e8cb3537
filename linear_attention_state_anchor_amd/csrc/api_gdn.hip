// C ABI: version, status strings and the gated-delta-rule replay entry point.
// Arguments are validated on the host; nothing is enqueued on failure.
#include <stdint.h>

#include "sr_internal.hpp"

extern "C" {

const char* sr_version(void) { return "sr_replay 0.1.0 (gfx950)"; }

const char* sr_status_str(int status) {
  switch (status) {
    case SR_OK: return "ok";
    case SR_EINVAL: return "invalid argument (null pointer, bad flag or misaligned buffer)";
    case SR_ESHAPE: return "unsupported or inconsistent shape";
    case SR_EDTYPE: return "unsupported dtype";
    case SR_EWORKSPACE: return "workspace missing or too small";
    case SR_ELAUNCH: return "kernel launch failed";
    case SR_EDEVICE: return "no usable device";
    default: return "unknown status";
  }
}

int sr_gdn_replay_state(const sr_gdn_desc* d, const sr_gdn_io* io, void* stream) {
  if (!d || !io) return SR_EINVAL;
  if (d->n_seqs < 0 || d->total_tokens < 0 || d->h_k < 1 || d->h_v < 1 || d->d_k < 1 ||
      d->d_v < 1 || d->h_v % d->h_k != 0)
    return SR_ESHAPE;
  auto dt_ok = [](int t) { return t == SR_BF16 || t == SR_F16 || t == SR_F32; };
  if (!dt_ok(d->dtype_qkv) || !dt_ok(d->dtype_o)) return SR_EDTYPE;
  if ((d->erase != 0 && d->erase != 1) || (d->alpha_is_log != 0 && d->alpha_is_log != 1))
    return SR_EINVAL;
  if (d->n_seqs == 0) return SR_OK;
  if (!io->cu_seqlens || !io->final_state) return SR_EINVAL;
  if (d->total_tokens > 0 && (!io->k || !io->v || !io->alpha)) return SR_EINVAL;
  if (io->o && d->total_tokens > 0 && !io->q) return SR_EINVAL;
  const int64_t grid = static_cast<int64_t>(d->n_seqs) * d->h_v;
  if (grid > INT32_MAX) return SR_ESHAPE;

  sr::GdnArgs a;
  a.n_seqs = d->n_seqs;
  a.total_tokens = d->total_tokens;
  a.h_k = d->h_k;
  a.h_v = d->h_v;
  a.d_k = d->d_k;
  a.d_v = d->d_v;
  a.dtype_qkv = d->dtype_qkv;
  a.dtype_o = d->dtype_o;
  a.erase = d->erase;
  a.alpha_is_log = d->alpha_is_log;
  a.scale = d->scale;
  a.q = io->q;
  a.k = io->k;
  a.v = io->v;
  a.alpha = io->alpha;
  a.beta = io->beta;
  a.cu = io->cu_seqlens;
  a.s0 = io->initial_state;
  a.s_out = io->final_state;
  a.o = io->o;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (d->dtype_qkv != SR_F32 && sr::gdn_chunk_supports(d->dtype_qkv, d->d_k, d->d_v)) {
    // the chunked kernel reads 16-byte rows of q, k and v
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    if (!al16(a.k) || !al16(a.v) || (a.o && !al16(a.q))) return SR_EINVAL;
    // outputs are written 4 values at a time
    const uintptr_t omask = d->dtype_o == SR_F32 ? 15u : 7u;
    if (a.o && (reinterpret_cast<uintptr_t>(a.o) & omask) != 0) return SR_EINVAL;
    e = sr::launch_gdn_chunk(a, s);
  } else if (sr::gdn_serial_supports(d->d_k, d->d_v)) {
    e = sr::launch_gdn_serial(a, s);
  } else {
    return SR_ESHAPE;
  }
  return e == hipSuccess ? SR_OK : SR_ELAUNCH;
}

}  // extern "C"
