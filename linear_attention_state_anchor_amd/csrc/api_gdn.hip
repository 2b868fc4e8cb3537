// C ABI: version, status strings and the gated-delta-rule replay entry point.
// Arguments are validated on the host; nothing is enqueued on failure.
#include <stdint.h>

#include "sr_internal.hpp"

namespace sr {

int validate_gdn(const sr_gdn_desc* d, const sr_gdn_io* io, GdnArgs* out) {
  if (!d || !io) return SR_EINVAL;
  if (d->n_seqs < 0 || d->total_tokens < 0 || d->h_k < 1 || d->h_v < 1 || d->d_k < 1 ||
      d->d_v < 1 || d->h_v % d->h_k != 0)
    return SR_ESHAPE;
  auto dt_ok = [](int t) { return t == SR_BF16 || t == SR_F16 || t == SR_F32; };
  if (!dt_ok(d->dtype_qkv) || !dt_ok(d->dtype_o)) return SR_EDTYPE;
  if ((d->erase != 0 && d->erase != 1) || (d->alpha_is_log != 0 && d->alpha_is_log != 1))
    return SR_EINVAL;
  const int64_t grid = static_cast<int64_t>(d->n_seqs) * d->h_v;
  if (grid > INT32_MAX) return SR_ESHAPE;
  const bool chunked = d->dtype_qkv != SR_F32 && gdn_chunk_supports(d->dtype_qkv, d->d_k, d->d_v);
  // chunked matrix-core kernel for 16-bit inputs with d in {64, 128}; the
  // token-serial kernel for everything else it supports
  if (!chunked && !gdn_serial_supports(d->d_k, d->d_v)) return SR_ESHAPE;
  if (d->n_seqs == 0) {
    *out = GdnArgs{};
    out->n_seqs = 0;
    return SR_OK;
  }
  if (!io->cu_seqlens || !io->final_state) return SR_EINVAL;
  if (d->total_tokens > 0 && (!io->k || !io->v || !io->alpha)) return SR_EINVAL;
  if (io->o && d->total_tokens > 0 && !io->q) return SR_EINVAL;
  GdnArgs& a = *out;
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
  if (chunked) {
    // the chunked kernel reads 16-byte rows of q, k and v
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    if (!al16(a.k) || !al16(a.v) || (a.o && !al16(a.q))) return SR_EINVAL;
    // outputs are written 4 values at a time
    const uintptr_t omask = d->dtype_o == SR_F32 ? 15u : 7u;
    if (a.o && (reinterpret_cast<uintptr_t>(a.o) & omask) != 0) return SR_EINVAL;
  }
  return SR_OK;
}

}  // namespace sr

extern "C" {

const char* sr_version(void) { return "sr_replay 0.2.0 (gfx950)"; }

const char* sr_status_str(int status) {
  switch (status) {
    case SR_OK: return "ok";
    case SR_EINVAL: return "invalid argument (null pointer, bad flag or misaligned buffer)";
    case SR_ESHAPE: return "unsupported or inconsistent shape";
    case SR_EDTYPE: return "unsupported dtype";
    case SR_EWORKSPACE: return "workspace missing or too small";
    case SR_ELAUNCH: return "kernel launch failed";
    case SR_EDEVICE: return "no usable device";
    case SR_EDATA: return "device-side inputs break a documented precondition";
    default: return "unknown status";
  }
}

size_t sr_gdn_workspace_bytes(const sr_gdn_desc* d) {
  sr_gdn_io io{};
  sr::GdnArgs a{};
  if (!d) return static_cast<size_t>(-1);
  // shape-level checks only (pointers are not known here)
  sr_gdn_desc probe = *d;
  probe.n_seqs = 0;
  return sr::validate_gdn(&probe, &io, &a) == SR_OK ? 0 : static_cast<size_t>(-1);
}

int sr_check_replay_inputs(const sr_gdn_desc* d, const sr_gdn_io* io, void* stream) {
  sr::GdnArgs a{};
  const int st = sr::validate_gdn(d, io, &a);
  if (st != SR_OK || a.n_seqs == 0) return st;
  return sr::check_replay(a, static_cast<hipStream_t>(stream));
}

int sr_gdn_replay_state(const sr_gdn_desc* d, const sr_gdn_io* io, void* workspace,
                        size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;  // no shape needs a workspace
  sr::GdnArgs a{};
  const int st = sr::validate_gdn(d, io, &a);
  if (st != SR_OK || a.n_seqs == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (sr::debug_checks_enabled()) {
    const int c = sr::check_replay(a, s);
    if (c != SR_OK) return c;
  }
  hipError_t e;
  if (a.dtype_qkv != SR_F32 && sr::gdn_chunk_supports(a.dtype_qkv, a.d_k, a.d_v))
    e = sr::launch_gdn_chunk(a, s);
  else
    e = sr::launch_gdn_serial(a, s);
  return e == hipSuccess ? SR_OK : SR_ELAUNCH;
}

}  // extern "C"
