// C ABI of the VLA scan library: argument validation and kernel dispatch.
// Every check runs before any launch; nothing here allocates device memory.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/vla.h"
#include "vla_kernels.h"
#include "vla_wide.h"
#include "vla_residual.h"

namespace {

thread_local std::string g_last_error;

// Event pairs of the chain-kernel timing hook (see vla_timing_enable).
struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> start, stop;
  int used = 0;
};
Timing& timing() {
  static Timing t;
  return t;
}
void timing_release(Timing& t) {
  for (hipEvent_t e : t.start) (void)hipEventDestroy(e);
  for (hipEvent_t e : t.stop) (void)hipEventDestroy(e);
  t.start.clear();
  t.stop.clear();
  t.used = 0;
  t.on = false;
}

// A side stream per device (default priority, non-blocking) and the events
// that order the state pass's parallel kernels on it against the chain
// kernel segments on the caller's stream.  Created on first use and kept
// until the process ends; enqueueing on them is serialised by the mutex.
constexpr int kMaxChainSegs = 16;
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t ev[2 * kMaxChainSegs + 2] = {};
  int side_wg = 0;   // workgroups of a prep or readout launch beside the chain kernel
  int ncu = 0;       // compute units of the device
  bool ready = false;
};
struct SidePool {
  std::mutex mu;
  SideStream dev[64];
};
SidePool& side_pool() {
  static SidePool p;
  return p;
}
// Needs side_pool().mu held; nullptr (and the HIP error in *err) on failure.
SideStream* side_stream(hipError_t* err) {
  int dev = 0;
  if ((*err = hipGetDevice(&dev)) != hipSuccess) return nullptr;
  if (dev < 0 || dev >= 64) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  SideStream& ss = side_pool().dev[dev];
  if (!ss.ready) {
    int ncu = 0;
    if ((*err = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return nullptr;
    // Five eighths of the compute units: the side work still keeps ahead of
    // the chain kernel, which loses a quarter of its speed to a full-width
    // side launch (measured on the 16-chain, 65536-token workload).
    ss.side_wg = std::max(1, ncu * 5 / 8);
    ss.ncu = ncu;
    if ((*err = hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking)) != hipSuccess) return nullptr;
    for (hipEvent_t& e : ss.ev)
      if ((*err = hipEventCreateWithFlags(&e, hipEventDisableTiming)) != hipSuccess) return nullptr;
    ss.ready = true;
  }
  *err = hipSuccess;
  return &ss;
}

// Blocks per chain-kernel segment for nblk blocks of 64 tokens: seg_blocks
// (default 256; < 0: all in one) rounded up to a multiple of 4, and large
// enough for at most kMaxChainSegs segments (a launch per segment costs a few
// microseconds).
int chain_segment_len(int nblk, int seg_blocks) {
  if (seg_blocks < 0 || seg_blocks > 2 * nblk) seg_blocks = 2 * nblk;
  if (seg_blocks == 0) seg_blocks = 256;
  seg_blocks = std::max(seg_blocks, (nblk + kMaxChainSegs - 2) / (kMaxChainSegs - 1));
  return (seg_blocks + 3) & ~3;
}

// Segment boundaries bnd[0] = 0 < ... < bnd[n] = nblk of the state pass; returns
// n.  Segment s's chain kernel runs beside the next segment's prep and the
// previous one's readout, so neighbours must not be much longer than it:
// the first segment is five eighths of a segment (its prep runs alone on the
// chip before the chain kernel, while the second segment's prep runs beside
// it), and a remainder under half a segment is shared with the segment
// before it so that the last one stays at least half a segment long (the
// readout of the one before runs beside it).
int chain_segments(int nblk, int seg_blocks, int* bnd) {
  const int len = chain_segment_len(nblk, seg_blocks);
  const int first = std::max(2, (len * 5 / 8 + 1) & ~1);
  int n = 0;
  bnd[n++] = 0;
  if (nblk <= first) {
    bnd[n++] = nblk;
    return n - 1;
  }
  bnd[n++] = first;
  const int rest = nblk - first, full = rest / len, rem = rest % len;
  const bool share = full >= 1 && rem > 0 && rem < len / 2;
  for (int i = 0; i < full - (share ? 1 : 0); ++i) bnd[n] = bnd[n - 1] + len, ++n;
  if (share) {
    bnd[n] = bnd[n - 1] + len / 2 + rem, ++n;
    bnd[n] = bnd[n - 1] + len / 2, ++n;
  } else if (rem > 0) {
    bnd[n] = bnd[n - 1] + rem, ++n;
  }
  return n - 1;
}

// Scratch of vla_scan_forward_noalloc: one static array per device, held
// until the process ends.  Host code never uses the array's name as an
// address: the device address comes from hipGetSymbolAddress, looked up once
// per device with that device current, and is kept here.
__device__ __align__(256) unsigned char scratch[VLA_NOALLOC_SCRATCH_BYTES];
struct ScratchTable {
  std::mutex mu;
  void* ptr[64] = {};
};
ScratchTable& scratch_table() {
  static ScratchTable t;
  return t;
}

vla_status_t fail(vla_status_t s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
vla_status_t fail(vla_status_t s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

vla_status_t hip_fail(hipError_t e, const char* what) {
  return fail(VLA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool supported_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

size_t dtype_size(int32_t t) { return t == VLA_BF16 ? 2 : 4; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// True when byte ranges [a, a+na) and [b, b+nb) intersect.
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// An output may alias its own input exactly, and must not partly overlap
// anything else it is checked against.
bool bad_alias(const void* out, size_t n_out, const void* in, size_t n_in, bool exact_ok) {
  if (exact_ok && out == in) return false;
  return overlap(out, n_out, in, n_in);
}

constexpr size_t kValidateBytes = 256;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Whether q, k, v come as strided views (any stride set) rather than contiguous.
bool strided(const vla_scan_params_t* p) { return p->stride_b != 0 || p->stride_h != 0 || p->stride_t != 0; }

// Bytes from the first to one past the last element a [B, H, T, d] view
// touches: the contiguous size, or the strided extent.
size_t seq_extent(const vla_scan_params_t* p, size_t es) {
  const size_t n_tok = static_cast<size_t>(p->B) * p->H * p->T;
  if (n_tok == 0) return 0;
  if (!strided(p)) return n_tok * p->d * es;
  const uint64_t last = static_cast<uint64_t>(p->B - 1) * p->stride_b + static_cast<uint64_t>(p->H - 1) * p->stride_h +
                        static_cast<uint64_t>(p->T - 1) * p->stride_t + p->d;
  return static_cast<size_t>(last) * es;
}

// Shape of a chunked run and the workspace layout it uses.
struct ChunkLayout {
  bool use = false;
  int L = 0, nchunks = 0, nperiods = 0, o = 0, q = 0;
  int nblk = 0;   // 64-token blocks of the state pass
  size_t off_A = 0, off_S = 0, off_n = 0, off_info = 0, off_G = 0, off_Gpre = 0, off_Gtot = 0, off_ND = 0, off_Ac = 0,
         off_alpha = 0, off_K = 0, off_Kx = 0, off_VT = 0, off_AT = 0, off_X = 0, off_wsig = 0, off_ld = 0, off_nb = 0,
         off_ncarry = 0, off_cnt = 0, off_flag = 0, off_gather = 0,
         total = 0;
  // Parallel-in-time state pass (additive update): segments per chain, and
  // its segment starts, segment ends, records, normalisers and flags.
  int para = 1;
  size_t off_pSit = 0, off_pF = 0, off_prec = 0, off_pn = 0, off_pconv = 0, off_pact = 0, off_pP = 0;
  // Residual update's state pass (replaces the additive one's buffers).
  size_t off_rW = 0, off_rU = 0, off_rN = 0, off_rQ = 0, off_rks = 0, off_rS = 0, off_rnb = 0, off_rnc = 0, off_rex = 0;
  // d = 128: the linear state pass's chunk sums (then chunk starts) of S and n.
  int ncs = 0;
  size_t off_lS = 0, off_ln = 0;
};

// Whether the d = 128 time-parallel schedule applies: its state pass is the
// plain prefix sum, valid only without the cap, for the additive update, and
// its kernels read bf16 storage.
bool linear_d128(const vla_scan_params_t* p) {
  const bool cap_on = p->s_cap > 0.f && std::isfinite(p->s_cap);
  return p->d == 128 && p->in_dtype == VLA_BF16 && p->update == VLA_UPDATE_ADDITIVE && !cap_on;
}

// Whether the chunked schedule can run these parameters with chunk length L.
bool chunk_len_fits(const vla_scan_params_t* p, int L) {
  if (L < 16 || L % 16 != 0) return false;
  if (p->nudge_period > 0 && p->nudge_period % L != 0) return false;
  return p->t0 % L == 0;
}

// The regions every schedule may add at the end: contiguous copies of
// strided q, k, v, then the validation flag.
ChunkLayout finish_layout(const vla_scan_params_t* p, ChunkLayout cl, size_t off) {
  if (strided(p)) {
    cl.off_gather = off;
    off = align_up(off + 3 * static_cast<size_t>(p->B) * p->H * p->T * p->d * dtype_size(p->in_dtype));
  }
  cl.off_flag = off;
  if (p->validate) off += kValidateBytes;
  cl.total = off;
  return cl;
}

// Chunks per workgroup of the d = 128 blocked inverse pass: the largest of
// 1, 2, 4, 8 that keeps at least 512 spans over all chains (two workgroups
// per compute unit).  Wide workload (2048 chunks of 512 tokens), ms per
// scan: spans of one chunk 5.67, two 5.53, four 5.42.
int inverse_span_chunks(int64_t chains, int nchunks) {
  int cm = 1;
  while (cm < 8 && chains * ((nchunks + 2 * cm - 1) / (2 * cm)) >= 512) cm *= 2;
  return cm;
}

// Segments of the parallel-in-time state pass: enough to give every chain's
// segments a compute unit of the 256 (one chain-kernel workgroup fills one),
// at most 16, and at least two blocks each; 1 keeps one pass per chain.
int para_segments(const vla_scan_params_t* p, int64_t chains, int nblk) {
  if (p->update != VLA_UPDATE_ADDITIVE || chains <= 0) return 1;
  int64_t G = p->para_segments;
  // By default one workgroup per compute unit, and segments of at least 8
  // blocks: a pass and a sweep cost a few microseconds of launches and
  // setup, so short chains gain little from more segments (32 chains of 32
  // blocks: 0.427 ms in one pass, 0.422 with two segments, 0.403 with four,
  // 0.424 with eight).
  if (G == 0) G = std::min<int64_t>(std::min<int64_t>(vla::kMaxParaSegs, 256 / chains), nblk / 8);
  G = std::min<int64_t>(G, std::min<int64_t>(vla::kMaxParaSegs, nblk / 2));
  return G >= 2 ? static_cast<int>(G) : 1;
}

ChunkLayout plan_schedule(const vla_scan_params_t* p) {
  ChunkLayout cl;
  const int64_t chains = static_cast<int64_t>(p->B) * p->H;
  // Grids of the chunked kernels hold one workgroup per 64-token block of
  // every chain (at most 256 threads each, below HIP's 2^32 work-items per
  // launch dimension); longer problems take the sequential schedule.
  constexpr int64_t kMaxBlocks = int64_t{1} << 22;
  const bool possible = (p->d == 64 || linear_d128(p)) && p->T > 0 && chains > 0 &&
                        chains * ((p->T + int64_t{63}) / 64) <= kMaxBlocks;
  int L = 0;
  if (possible) {
    if (p->chunk_len > 0) {
      if (chunk_len_fits(p, p->chunk_len)) L = p->chunk_len;
    } else {
      // The longest chunk that still gives at least kMinChunks chunks over
      // all chains (the inverse pass keeps the SIMDs busy only with many
      // chunks side by side), else the shortest that fits: 512 tokens for 16
      // chains of 65536 and for 128 chains of 8192, 64 for 32 chains of
      // 2048 (0.42 against 0.46 ms with 128 and 0.61 with 256).
      constexpr int64_t kMinChunks = 1024;
      for (int cand : {512, 256, 128, 64}) {
        if (!chunk_len_fits(p, cand)) continue;
        L = cand;
        if (chains * ((p->T + cand - 1) / cand) >= kMinChunks) break;
      }
    }
  }
  bool use = false;
  if (p->schedule == VLA_SCHEDULE_CHUNKED) {
    use = L > 0;
  } else if (p->schedule == VLA_SCHEDULE_AUTO && L > 0) {
    // Few chains leave most compute units idle in the sequential schedule;
    // chunking pays once every chain has several chunks.
    const int64_t nch = (p->T + L - 1) / L;
    use = chains <= 256 && nch >= 8;
  }
  size_t off = 0;
  if (use) {
    cl.use = true;
    cl.L = L;
    cl.nchunks = (p->T + L - 1) / L;
    cl.o = static_cast<int>(p->t0 / L);
    cl.q = p->nudge_period > 0 ? p->nudge_period / L : 0;
    // Periods touched: 1 + nudges at the ends of chunks 0 .. nchunks-2.
    cl.nperiods = 1 + (cl.q > 0 ? (cl.o + cl.nchunks - 1) / cl.q - cl.o / cl.q : 0);
    if (p->d == 128) {
      // Inverse side as at d = 64 (matrices of 128 x 128), then the linear
      // state pass's chunk sums.
      const size_t d = 128, d2 = d * d, C = static_cast<size_t>(chains), nch = cl.nchunks;
      cl.ncs = (p->T + vla::kLinChunk - 1) / vla::kLinChunk;
      cl.off_A = off; off = align_up(off + C * d2 * 4);
      cl.off_S = off; off = align_up(off + C * d2 * 4);
      cl.off_n = off; off = align_up(off + C * d * 4);
      cl.off_info = off; off = align_up(off + C * 4 * 4);
      cl.off_G = off; off = align_up(off + C * nch * d2 * 4);
      cl.off_Gpre = off; off = align_up(off + C * nch * d2 * 8);
      cl.off_Gtot = off; off = align_up(off + C * static_cast<size_t>(cl.nperiods) * d2 * 8);
      cl.off_ND = off; off = align_up(off + C * static_cast<size_t>(cl.nperiods) * 2 * d2 * 8);
      cl.off_Ac = off; off = align_up(off + C * nch * d2 * 4);
      cl.off_alpha = off; off = align_up(off + C * static_cast<size_t>(p->T) * d * 4);
      cl.off_lS = off; off = align_up(off + C * static_cast<size_t>(cl.ncs) * d2 * 4);
      cl.off_ln = off; off = align_up(off + C * static_cast<size_t>(cl.ncs) * d * 4);
      return finish_layout(p, cl, off);
    }
    const size_t d2 = 64 * 64, C = static_cast<size_t>(chains), nch = cl.nchunks;
    cl.off_A = off; off = align_up(off + C * d2 * 4);
    cl.off_S = off; off = align_up(off + C * d2 * 4);
    cl.off_n = off; off = align_up(off + C * 64 * 4);
    cl.off_info = off; off = align_up(off + C * 4 * 4);
    cl.off_G = off; off = align_up(off + C * nch * d2 * 4);
    cl.off_Gpre = off; off = align_up(off + C * nch * d2 * 8);
    cl.off_Gtot = off; off = align_up(off + C * static_cast<size_t>(cl.nperiods) * d2 * 8);
    cl.off_ND = off; off = align_up(off + C * static_cast<size_t>(cl.nperiods) * 2 * d2 * 8);
    cl.off_Ac = off; off = align_up(off + C * nch * d2 * 4);
    cl.off_alpha = off; off = align_up(off + C * static_cast<size_t>(p->T) * 64 * 4);
    cl.nblk = (p->T + 63) / 64;
    const size_t nb = cl.nblk, T = static_cast<size_t>(p->T);
    if (p->update == VLA_UPDATE_RESIDUAL) {
      cl.off_rW = off; off = align_up(off + C * nb * d2 * 4);
      cl.off_rU = off; off = align_up(off + C * nb * d2 * 4);
      cl.off_rN = off; off = align_up(off + C * nb * 3 * d2 * 2);
      cl.off_rQ = off; off = align_up(off + C * nb * d2 * 4);
      cl.off_rks = off; off = align_up(off + C * nb * 64 * 4);
      cl.off_rS = off; off = align_up(off + C * nb * d2 * 4);
      cl.off_rnb = off; off = align_up(off + C * nb * 64 * 4);
      cl.off_rnc = off; off = align_up(off + 2 * C * 64 * 4);   // normaliser carries between segments
      cl.off_rex = off; off = align_up(off + C * nb * 4);       // per-block exact cap-test flags
      return finish_layout(p, cl, off);
    }
    cl.para = para_segments(p, chains, cl.nblk);
    if (cl.para > 1) {
      const size_t G = static_cast<size_t>(cl.para);
      cl.off_pSit = off; off = align_up(off + C * G * d2 * 4);
      cl.off_pF = off; off = align_up(off + C * G * d2 * 4);
      cl.off_prec = off; off = align_up(off + C * G * 4 * 4);
      cl.off_pn = off; off = align_up(off + C * G * 64 * 4);
      cl.off_pconv = off; off = align_up(off + C * 4);
      cl.off_pact = off; off = align_up(off + C * G * 4);
      cl.off_pP = off; off = align_up(off + C * G * vla::kParaSub * d2 * 4);
    }
    cl.off_K = off; off = align_up(off + C * nb * 2304 * 4);
    cl.off_Kx = off; off = align_up(off + C * nb * d2 * 4);
    // Regrouped update operands: fp32 storage only (bf16 reads its LDS rows).
    const size_t nreg = p->in_dtype == VLA_BF16 ? 0 : C * nb * d2;
    cl.off_VT = off; off = align_up(off + nreg * 4);
    cl.off_AT = off; off = align_up(off + nreg * 4);
    cl.off_X = off; off = align_up(off + C * nb * d2 * 4);
    cl.off_wsig = off; off = align_up(off + C * T * 2 * 4);
    cl.off_ld = off; off = align_up(off + C * T * 4);
    cl.off_nb = off; off = align_up(off + C * nb * 64 * 4);
    cl.off_ncarry = off; off = align_up(off + C * 64 * 4);
    cl.off_cnt = off; off = align_up(off + C * 2 * 4);
  }
  return finish_layout(p, cl, off);
}

vla_status_t check_params(const vla_scan_params_t* p) {
  if (!p) return fail(VLA_EINVAL, "params is NULL");
  if (p->B < 0 || p->H < 0 || p->T < 0)
    return fail(VLA_EINVAL, "B, H, T must be >= 0 (got %d, %d, %d)", p->B, p->H, p->T);
  if (!supported_d(p->d)) return fail(VLA_EUNSUPPORTED, "d = %d unsupported (16, 32, 64, 128)", p->d);
  if (p->r < 1 || p->r > 4) return fail(VLA_EUNSUPPORTED, "r = %d unsupported (1..4)", p->r);
  if (p->in_dtype != VLA_F32 && p->in_dtype != VLA_BF16)
    return fail(VLA_EUNSUPPORTED, "in_dtype %d unsupported", static_cast<int>(p->in_dtype));
  if (!(p->eps >= 0.f) || !std::isfinite(p->eps)) return fail(VLA_EINVAL, "eps must be finite and >= 0");
  if (p->nudge_period < 0) return fail(VLA_EINVAL, "nudge_period must be >= 0");
  if (!std::isfinite(p->den_eps)) return fail(VLA_EINVAL, "den_eps must be finite");
  if (std::isnan(p->s_cap)) return fail(VLA_EINVAL, "s_cap is NaN");
  if (p->t0 < 0) return fail(VLA_EINVAL, "t0 must be >= 0");
  if (p->schedule != VLA_SCHEDULE_AUTO && p->schedule != VLA_SCHEDULE_SEQUENTIAL &&
      p->schedule != VLA_SCHEDULE_CHUNKED)
    return fail(VLA_EUNSUPPORTED, "schedule %d unsupported", p->schedule);
  if (p->chunk_len < 0) return fail(VLA_EINVAL, "chunk_len must be >= 0");
  if (p->update != VLA_UPDATE_ADDITIVE && p->update != VLA_UPDATE_RESIDUAL)
    return fail(VLA_EUNSUPPORTED, "update %d unsupported", p->update);
  if (p->para_segments < 0 || p->para_segments > vla::kMaxParaSegs)
    return fail(VLA_EINVAL, "para_segments must be 0..%d (got %d)", vla::kMaxParaSegs, p->para_segments);
  const int64_t chains = static_cast<int64_t>(p->B) * p->H;
  if (chains > 0x7fffffff) return fail(VLA_EUNSUPPORTED, "B*H too large");
  if (strided(p)) {
    const int64_t es = static_cast<int64_t>(dtype_size(p->in_dtype));
    if (p->stride_b < 0 || p->stride_h < 0 || p->stride_t < 0)
      return fail(VLA_EINVAL, "strides must be >= 0 (got %lld, %lld, %lld)", static_cast<long long>(p->stride_b),
                  static_cast<long long>(p->stride_h), static_cast<long long>(p->stride_t));
    if (p->T > 1 && p->stride_t < p->d) return fail(VLA_EINVAL, "stride_t must be >= d when T > 1");
    if ((p->stride_b * es) % 16 || (p->stride_h * es) % 16 || (p->stride_t * es) % 16)
      return fail(VLA_EINVAL, "strides times the element size must be multiples of 16 bytes");
    const int64_t lim = static_cast<int64_t>(1) << 50;
    if (p->stride_b > lim || p->stride_h > lim || p->stride_t > lim) return fail(VLA_EUNSUPPORTED, "strides too large");
  }
  return VLA_OK;
}

}  // namespace

extern "C" {

void vla_scan_params_init(vla_scan_params_t* p) {
  if (!p) return;
  std::memset(p, 0, sizeof(*p));
  p->d = 64;
  p->r = 1;
  p->in_dtype = VLA_F32;
  p->eps = 1e-6f;
  p->nudge_period = 0;
  p->s_cap = 0.f;
  p->den_eps = 1e-6f;
  p->t0 = 0;
  p->schedule = VLA_SCHEDULE_AUTO;
  p->validate = 0;
  p->chunk_len = 0;
  p->segment_blocks = 0;
  p->update = VLA_UPDATE_ADDITIVE;
}

vla_status_t vla_scan_workspace_size(const vla_scan_params_t* p, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(VLA_EINVAL, "bytes is NULL");
  const vla_status_t s = check_params(p);
  if (s != VLA_OK) return s;
  if (p->schedule == VLA_SCHEDULE_CHUNKED && !plan_schedule(p).use)
    return fail(VLA_EUNSUPPORTED, "chunked schedule needs d = 64 (or d = 128 with bf16 storage, the additive "
                                  "update and no cap), T > 0 and a chunk length dividing nudge_period and t0");
  *bytes = plan_schedule(p).total;
  return VLA_OK;
}

vla_status_t vla_scan_forward(const vla_scan_params_t* p, const void* q, const void* k, const void* v,
                              const void* u, const float* A0, const float* S0, const float* n0, void* o,
                              float* A_T, float* S_T, float* n_T, int32_t* stats, void* workspace,
                              size_t workspace_bytes, void* stream_ptr) {
  g_last_error.clear();
  vla_status_t s = check_params(p);
  if (s != VLA_OK) return s;
  const int64_t chains = static_cast<int64_t>(p->B) * p->H;
  const int d = p->d, r = p->r;
  const size_t es = dtype_size(p->in_dtype);
  const size_t n_tok = static_cast<size_t>(chains) * static_cast<size_t>(p->T);
  const size_t b_seq = n_tok * d * es, b_u = b_seq * r;
  const size_t b_in = seq_extent(p, es);   // bytes each of q, k, v spans (strided or not)
  const size_t b_mat = static_cast<size_t>(chains) * d * d * sizeof(float);
  const size_t b_vec = static_cast<size_t>(chains) * d * sizeof(float);
  if (static_cast<uint64_t>(n_tok) * r * d > (1ull << 62)) return fail(VLA_EUNSUPPORTED, "problem too large");

  if (chains == 0) return VLA_OK;
  if (n_tok > 0 && (!q || !k || !v || !u || !o)) return fail(VLA_EINVAL, "q, k, v, u and o must be non-NULL");
  if (!A_T || !S_T || !n_T) return fail(VLA_EINVAL, "A_T, S_T and n_T must be non-NULL");
  const void* seq[5] = {q, k, v, u, o};
  for (const void* x : seq)
    if (n_tok > 0 && !aligned(x, 16)) return fail(VLA_EINVAL, "q, k, v, u, o must be 16-byte aligned");
  if (!aligned(A0, 16) || !aligned(S0, 16) || !aligned(A_T, 16) || !aligned(S_T, 16))
    return fail(VLA_EINVAL, "A0, S0, A_T, S_T must be 16-byte aligned");
  if (!aligned(n0, 4) || !aligned(n_T, 4)) return fail(VLA_EINVAL, "n0, n_T must be 4-byte aligned");

  // Aliasing: outputs may alias only their own initial state, exactly.
  const struct { const void* p; size_t n; } ins[] = {{q, b_in}, {k, b_in}, {v, b_in}, {u, b_u}};
  const struct { const void* p; size_t n; const void* own; } outs[] = {
      {o, b_seq, nullptr}, {A_T, b_mat, A0}, {S_T, b_mat, S0}, {n_T, b_vec, n0},
      {stats, static_cast<size_t>(chains) * 16, nullptr}};
  const int n_outs = static_cast<int>(sizeof(outs) / sizeof(outs[0]));
  for (int oi = 0; oi < n_outs; ++oi) {
    const auto& ot = outs[oi];
    if (!ot.p) continue;
    for (const auto& in : ins)
      if (bad_alias(ot.p, ot.n, in.p, in.n, false)) return fail(VLA_EINVAL, "an output overlaps q, k, v or u");
    const struct { const void* p; size_t n; } st[] = {{A0, b_mat}, {S0, b_mat}, {n0, b_vec}};
    for (const auto& sx : st)
      if (bad_alias(ot.p, ot.n, sx.p, sx.n, ot.own == sx.p)) return fail(VLA_EINVAL, "outputs overlap the state");
    for (int oj = oi + 1; oj < n_outs; ++oj)
      if (overlap(ot.p, ot.n, outs[oj].p, outs[oj].n)) return fail(VLA_EINVAL, "outputs overlap each other");
  }

  size_t need = 0;
  s = vla_scan_workspace_size(p, &need);
  if (s != VLA_OK) return s;
  if (workspace_bytes < need || (need > 0 && (!workspace || !aligned(workspace, kAlign))))
    return fail(VLA_EWORKSPACE, "workspace of %zu bytes (256-byte aligned) needed (got %zu)", need,
                workspace_bytes);
  const ChunkLayout cl = plan_schedule(p);
  if (need > 0 && overlap(workspace, need, A0, b_mat) + overlap(workspace, need, S0, b_mat) +
                        overlap(workspace, need, n0, b_vec) + overlap(workspace, need, q, b_in) +
                        overlap(workspace, need, k, b_in) + overlap(workspace, need, v, b_in) +
                        overlap(workspace, need, u, b_u) + overlap(workspace, need, o, b_seq) +
                        overlap(workspace, need, A_T, b_mat) + overlap(workspace, need, S_T, b_mat) +
                        overlap(workspace, need, n_T, b_vec) > 0)
    return fail(VLA_EINVAL, "workspace overlaps a tensor argument");

  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const bool bf16 = p->in_dtype == VLA_BF16;

  // Strided q, k, v: gathered into contiguous rows in the workspace, which
  // every kernel below then reads in place of the views.
  if (strided(p) && n_tok > 0) {
    vla::GatherArgs g{};
    g.q = static_cast<const char*>(q);
    g.k = static_cast<const char*>(k);
    g.v = static_cast<const char*>(v);
    g.dst = static_cast<char*>(workspace) + cl.off_gather;
    g.rows = static_cast<int64_t>(n_tok);
    g.T = p->T;
    g.H = p->H;
    g.stride_b = p->stride_b;
    g.stride_h = p->stride_h;
    g.stride_t = p->stride_t;
    g.elem_bytes = static_cast<int32_t>(es);
    g.row_bytes = static_cast<int32_t>(d * es);
    const hipError_t e = vla::launch_gather_rows(g, stream);
    if (e != hipSuccess) return hip_fail(e, "gather launch");
    q = g.dst;
    k = g.dst + b_seq;
    v = g.dst + 2 * b_seq;
  }

  if (p->validate && n_tok > 0) {
    int32_t* flag = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + cl.off_flag);
    hipError_t e = vla::launch_clear_flag(flag, stream);
    if (e != hipSuccess) return hip_fail(e, "validate");
    const int64_t n_seq = static_cast<int64_t>(n_tok) * d;
    const void* bufs[4] = {q, k, v, u};
    for (int i = 0; i < 4; ++i) {
      e = vla::launch_nonfinite_check(bufs[i], i == 3 ? n_seq * r : n_seq, bf16, flag, stream);
      if (e != hipSuccess) return hip_fail(e, "validate");
    }
    int32_t host_flag = 0;
    e = hipMemcpyAsync(&host_flag, flag, sizeof(host_flag), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "validate");
    if (host_flag) return fail(VLA_ENONFINITE, "an input holds NaN or Inf");
  }

  vla::ScanArgs a{};
  a.q = q; a.k = k; a.v = v; a.u = u;
  a.A0 = A0; a.S0 = S0; a.n0 = n0;
  a.o = o; a.A_T = A_T; a.S_T = S_T; a.n_T = n_T; a.stats = stats;
  a.T = p->T; a.r = r; a.eps = p->eps;
  a.nudge_period = p->nudge_period;
  a.nudge_phase0 = p->nudge_period > 0 ? static_cast<int32_t>((p->t0 + 1) % p->nudge_period) : 0;
  a.cap_on = (p->s_cap > 0.f && std::isfinite(p->s_cap)) ? 1 : 0;
  a.cap = a.cap_on ? p->s_cap : 0.f;
  a.den_eps = p->den_eps;
  a.residual = p->update == VLA_UPDATE_RESIDUAL ? 1 : 0;
  if (!cl.use) {
    const hipError_t e = vla::launch_scan_sequential(a, d, bf16, static_cast<int>(chains), nullptr, stream);
    if (e != hipSuccess) return hip_fail(e, "scan launch");
    return VLA_OK;
  }

  // Chunked schedule: prologue (state snapshot, Gram matrices, (N, D) chain,
  // chunk-start inverses), inverse pass per chunk, state pass per chain, and
  // the sequential fallback for any chain flagged on the way.
  char* ws = static_cast<char*>(workspace);
  vla::ChunkPlan pl{};
  pl.chains = static_cast<int>(chains);
  pl.T = p->T;
  pl.r = r;
  pl.d = d;
  pl.L = cl.L;
  pl.nchunks = cl.nchunks;
  pl.nperiods = cl.nperiods;
  pl.o = cl.o;
  pl.q = cl.q;
  pl.eps = p->eps;
  pl.A_init = reinterpret_cast<float*>(ws + cl.off_A);
  pl.S_init = reinterpret_cast<float*>(ws + cl.off_S);
  pl.n_init = reinterpret_cast<float*>(ws + cl.off_n);
  pl.chain_info = reinterpret_cast<int32_t*>(ws + cl.off_info);
  pl.G = reinterpret_cast<float*>(ws + cl.off_G);
  pl.Gpre = reinterpret_cast<double*>(ws + cl.off_Gpre);
  pl.Gtot = reinterpret_cast<double*>(ws + cl.off_Gtot);
  pl.ND = reinterpret_cast<double*>(ws + cl.off_ND);
  pl.Ac = reinterpret_cast<float*>(ws + cl.off_Ac);
  pl.alpha = reinterpret_cast<float*>(ws + cl.off_alpha);
  hipError_t e = vla::launch_chunk_prologue(pl, A0, S0, n0, u, bf16, stream);
  if (e != hipSuccess) return hip_fail(e, "chunked prologue launch");
  // Later passes read the snapshot, so outputs may alias the initial state.
  a.A0 = pl.A_init;
  a.S0 = pl.S_init;
  a.n0 = pl.n_init;
  vla::StatePlan sp{};
  sp.T = p->T;
  sp.nblk = cl.nblk;
  sp.bf16 = bf16 ? 1 : 0;
  sp.v = v;
  sp.alpha = pl.alpha;
  sp.Kmat = reinterpret_cast<float*>(ws + cl.off_K);
  sp.Kcross = reinterpret_cast<float*>(ws + cl.off_Kx);
  sp.VT = ws + cl.off_VT;
  sp.AT = reinterpret_cast<float*>(ws + cl.off_AT);
  sp.Xsnap = reinterpret_cast<float*>(ws + cl.off_X);
  sp.wsig = reinterpret_cast<float*>(ws + cl.off_wsig);
  sp.ld = reinterpret_cast<float*>(ws + cl.off_ld);
  sp.nblock = reinterpret_cast<float*>(ws + cl.off_nb);
  float* n_carry = reinterpret_cast<float*>(ws + cl.off_ncarry);
  int32_t* counters = reinterpret_cast<int32_t*>(ws + cl.off_cnt);

  // Chunk-start inverses and the inverse pass over all chunks at once.  The
  // pass keeps every SIMD busy only with all chunks side by side: on a part
  // of them (a segment's) it takes nearly as long, so it is not pipelined
  // with the chain kernel below.
  if (d == 128) {
    // The blocked pass at d = 128 takes spans of cm chunks per workgroup
    // (nudges at chunk ends are applied inside the span): each span needs
    // one start inverse, a 128 x 128 fp64 inversion (wide workload: 2048
    // chunks of 512 tokens in 512 spans of four).
    const int cm = inverse_span_chunks(chains, cl.nchunks);
    const int nspan = (cl.nchunks + cm - 1) / cm;
    if ((e = vla::launch_chunk_start128(pl, 0, nspan, cm, stream)) != hipSuccess)
      return hip_fail(e, "chunk-start launch");
    e = vla::launch_inverse_wy128(a, pl.Ac, pl.alpha, pl.chain_info, cl.L, cl.nchunks, cm, 0, nspan,
                                  static_cast<int>(chains), stream);
  } else if ((e = vla::launch_chunk_start(pl, 0, cl.nchunks, stream)) != hipSuccess) {
    return hip_fail(e, "chunk-start launch");
  } else if (p->r == 1 && d == 64)
    e = vla::launch_inverse_wy(a, pl.Ac, pl.alpha, pl.chain_info, cl.L, cl.nchunks, 0, cl.nchunks, bf16,
                               static_cast<int>(chains), stream);
  else
    e = vla::launch_scan_inverse_chunks(a, pl.Ac, pl.alpha, pl.chain_info, cl.L, cl.nchunks, 0, cl.nchunks, d, bf16,
                                        static_cast<int>(chains), stream);
  if (e != hipSuccess) return hip_fail(e, "chunked inverse launch");

  if (d == 128) {
    // Linear state pass (no cap), then the sequential rerun of any chain the
    // inverse side flagged.
    vla::LinPlan lp{};
    lp.chains = static_cast<int>(chains);
    lp.T = p->T;
    lp.ncs = cl.ncs;
    lp.q = q; lp.k = k; lp.v = v; lp.o = o;
    lp.alpha = pl.alpha;
    lp.dS = reinterpret_cast<float*>(ws + cl.off_lS);
    lp.dn = reinterpret_cast<float*>(ws + cl.off_ln);
    lp.S_init = pl.S_init;
    lp.n_init = pl.n_init;
    lp.S_T = S_T;
    lp.n_T = n_T;
    lp.chain_info = pl.chain_info;
    lp.stats = stats;
    lp.den_eps = p->den_eps;
    if ((e = vla::launch_linear_state(lp, stream)) != hipSuccess) return hip_fail(e, "linear state pass launch");
    e = vla::launch_scan_sequential(a, d, bf16, static_cast<int>(chains), pl.chain_info, stream);
    if (e != hipSuccess) return hip_fail(e, "chunked fallback launch");
    return VLA_OK;
  }

  if (p->update == VLA_UPDATE_RESIDUAL) {
    // Residual state pass: per-block affine maps of S, their chain, readout.
    vla::ResPlan rp{};
    rp.T = p->T;
    rp.nblk = cl.nblk;
    rp.bf16 = bf16 ? 1 : 0;
    rp.q = q; rp.k = k; rp.v = v; rp.o = o;
    rp.alpha = pl.alpha;
    rp.W = reinterpret_cast<float*>(ws + cl.off_rW);
    rp.U = reinterpret_cast<float*>(ws + cl.off_rU);
    rp.NTF = reinterpret_cast<uint16_t*>(ws + cl.off_rN);
    rp.QT = reinterpret_cast<float*>(ws + cl.off_rQ);
    rp.ksum = reinterpret_cast<float*>(ws + cl.off_rks);
    rp.Ssnap = reinterpret_cast<float*>(ws + cl.off_rS);
    rp.nblock = reinterpret_cast<float*>(ws + cl.off_rnb);
    rp.exact = reinterpret_cast<int32_t*>(ws + cl.off_rex);
    const int nch = static_cast<int>(chains);
    const int nblk = cl.nblk;
    // Segments as for the additive pass: the chain kernel runs them in order
    // on the caller's stream while the side stream preps the next one and
    // reads out the previous one.  The side kernels cannot share a compute
    // unit with the chain kernel (neither fits beside the other's LDS).
    int bnd[kMaxChainSegs + 1];
    const int nseg = chain_segments(nblk, p->segment_blocks, bnd);
    float* ncar[2] = {reinterpret_cast<float*>(ws + cl.off_rnc),
                      reinterpret_cast<float*>(ws + cl.off_rnc) + static_cast<size_t>(chains) * 64};
    auto nprefix = [&](int sidx, hipStream_t st) {
      const float* nin = sidx == 0 ? pl.n_init : ncar[(sidx - 1) & 1];
      float* nout = sidx + 1 == nseg ? n_T : ncar[sidx & 1];
      return vla::launch_res_nprefix(rp, bnd[sidx], bnd[sidx + 1], nin, nout, nch, st);
    };
    auto chain = [&](int sidx, hipStream_t st) {
      hipEvent_t ev0 = nullptr, ev1 = nullptr;
      {
        Timing& tm = timing();
        std::lock_guard<std::mutex> lock(tm.mu);
        if (tm.on && tm.used < VLA_TIMING_SLOTS) {
          ev0 = tm.start[tm.used];
          ev1 = tm.stop[tm.used];
          ++tm.used;
        }
      }
      const bool first = sidx == 0;
      const float* S_in = first ? pl.S_init : rp.Ssnap + static_cast<int64_t>(bnd[sidx]) * 64 * 64;
      const int64_t stride = first ? 64 * 64 : static_cast<int64_t>(nblk) * 64 * 64;
      return vla::launch_res_chain(rp, bnd[sidx], bnd[sidx + 1], S_in, stride, S_T, stats, pl.chain_info,
                                   sidx + 1 == nseg ? 1 : 0, nch, st, ev0, ev1);
    };
    if (nseg == 1) {
      if ((e = vla::launch_res_prep(rp, nch, 0, nblk, 0, stream)) != hipSuccess || (e = nprefix(0, stream)) != hipSuccess)
        return hip_fail(e, "residual prep launch");
      if ((e = chain(0, stream)) != hipSuccess) return hip_fail(e, "residual chain launch");
      if ((e = vla::launch_res_readout(rp, p->den_eps, a.cap, a.cap_on, nch, 0, nblk, 0, pl.chain_info, stream)) !=
          hipSuccess)
        return hip_fail(e, "residual readout launch");
    } else {
      std::lock_guard<std::mutex> lock(side_pool().mu);
      SideStream* ss = side_stream(&e);
      if (!ss) return hip_fail(e, "side stream setup");
      hipStream_t side = ss->stream;
      hipEvent_t ev_in = ss->ev[0], ev_end = ss->ev[1];
      hipEvent_t* ev_prep = ss->ev + 2;
      hipEvent_t* ev_chain = ss->ev + 2 + kMaxChainSegs;
      // A chain workgroup needs a whole compute unit, so each segment's chain
      // launch must find free units when it starts, which is also when the
      // previous segment's readout becomes ready: that readout is held to
      // (units - chains) workgroups, which leaves enough units empty.  The
      // next prep starts after the readout, when the chain kernel already
      // holds its units, and runs uncapped.  (Uncapped readouts kept the
      // chain's workgroups waiting: 2.85 against 1.93 ms of chain time per
      // scan on the 65536-token, 16-chain workload.)
      const int res_wg = std::max(1, ss->ncu - nch);
      auto prep = [&](int sidx) {
        hipError_t r = vla::launch_res_prep(rp, nch, bnd[sidx], bnd[sidx + 1] - bnd[sidx], 0, side);
        if (r == hipSuccess) r = nprefix(sidx, side);
        return r != hipSuccess ? r : hipEventRecord(ev_prep[sidx], side);
      };
      if ((e = hipEventRecord(ev_in, stream)) != hipSuccess || (e = hipStreamWaitEvent(side, ev_in, 0)) != hipSuccess ||
          (e = prep(0)) != hipSuccess)
        return hip_fail(e, "residual prep launch");
      for (int sidx = 0; sidx < nseg; ++sidx) {
        if (sidx + 1 < nseg && (e = prep(sidx + 1)) != hipSuccess) return hip_fail(e, "residual prep launch");
        if ((e = hipStreamWaitEvent(stream, ev_prep[sidx], 0)) != hipSuccess || (e = chain(sidx, stream)) != hipSuccess ||
            (e = hipEventRecord(ev_chain[sidx], stream)) != hipSuccess)
          return hip_fail(e, "residual chain launch");
        if ((e = hipStreamWaitEvent(side, ev_chain[sidx], 0)) != hipSuccess ||
            (e = vla::launch_res_readout(rp, p->den_eps, a.cap, a.cap_on, nch, bnd[sidx], bnd[sidx + 1] - bnd[sidx],
                                         sidx + 1 == nseg ? 0 : res_wg, pl.chain_info, side)) != hipSuccess)
          return hip_fail(e, "residual readout launch");
      }
      if ((e = hipEventRecord(ev_end, side)) != hipSuccess || (e = hipStreamWaitEvent(stream, ev_end, 0)) != hipSuccess)
        return hip_fail(e, "side stream join");
    }
    if ((e = vla::launch_stats_finalize(stats, pl.chain_info, nch, stream)) != hipSuccess)
      return hip_fail(e, "stats launch");
    vla::ResRestart rs{};
    rs.chunk_len = cl.L;
    rs.nchunks = cl.nchunks;
    rs.Ac = pl.Ac;
    rs.A_init = pl.A_init;
    rs.S_init = pl.S_init;
    rs.n_init = pl.n_init;
    rs.chain_info = pl.chain_info;
    if ((e = vla::launch_res_restart(rp, rs, nch, stream)) != hipSuccess) return hip_fail(e, "restart launch");
    e = vla::launch_scan_sequential(a, d, bf16, nch, pl.chain_info, stream);
    if (e != hipSuccess) return hip_fail(e, "chunked fallback launch");
    return VLA_OK;
  }

  // State pass: prep, the chain kernel, readout.  The sequence is cut into
  // segments (even block counts): the chain kernel runs them one after
  // another on the caller's stream while a side stream preps the next
  // segment and reads out the previous one, so only the first prep and the
  // last readout stay outside the chain kernel's time.  The side launches
  // between are held to a part of the chip (SideStream::side_wg).
  const int nblk = cl.nblk;
  int bnd[kMaxChainSegs + 1];
  const int nseg = chain_segments(nblk, p->segment_blocks, bnd);
  auto seg_lo = [&](int sidx) { return bnd[sidx]; };
  auto next_timing = [&](hipEvent_t* ev0, hipEvent_t* ev1) {
    Timing& tm = timing();
    std::lock_guard<std::mutex> lock(tm.mu);
    *ev0 = *ev1 = nullptr;
    if (tm.on && tm.used < VLA_TIMING_SLOTS) {
      *ev0 = tm.start[tm.used];
      *ev1 = tm.stop[tm.used];
      ++tm.used;
    }
  };
  auto chain_seg = [&](int sidx) {
    vla::ChainSeg sg{};
    sg.b_lo = seg_lo(sidx);
    sg.b_hi = seg_lo(sidx + 1);
    if (sidx == 0) {
      sg.S_in = pl.S_init;
      sg.S_in_stride = 64 * 64;
      sg.n_in = pl.n_init;
    } else {   // S and n where the previous segment left them
      sg.S_in = sp.Xsnap + static_cast<int64_t>(sg.b_lo) * 64 * 64;
      sg.S_in_stride = static_cast<int64_t>(nblk) * 64 * 64;
      sg.n_in = n_carry;
    }
    sg.n_in_stride = 64;
    sg.n_carry = n_carry;
    sg.counters = counters;
    sg.last = sg.b_hi == nblk ? 1 : 0;
    return sg;
  };
  const int nch = static_cast<int>(chains);
  if (cl.para > 1) {
    // Parallel in time: prep of every block, the plain sums over the
    // segments' sub-steps and the first sweep's guesses of the segment
    // starts, then passes of all segments from the swept starts until they
    // stop moving (at most kParaPasses; a chain that has not converged by
    // then is recomputed by the sequential fallback below), then the readout
    // of every block.
    constexpr int kParaPasses = 8;
    const int G = cl.para;
    vla::ParaPlan pp{};
    pp.chains = nch;
    pp.nseg = G;
    for (int sidx = 0; sidx <= G; ++sidx) pp.bnd[sidx] = static_cast<int>(static_cast<int64_t>(sidx) * nblk / G);
    pp.S_init = pl.S_init;
    pp.Sit = reinterpret_cast<float*>(ws + cl.off_pSit);
    pp.F = reinterpret_cast<float*>(ws + cl.off_pF);
    pp.rec = reinterpret_cast<float*>(ws + cl.off_prec);
    pp.conv = reinterpret_cast<int32_t*>(ws + cl.off_pconv);
    pp.chain_info = pl.chain_info;
    pp.cap = a.cap;
    pp.cap_on = a.cap_on;
    pp.active = reinterpret_cast<int32_t*>(ws + cl.off_pact);
    // Stop once no start moves by more than 4e-5 of its norm in a sweep: each
    // sweep shrinks the moves about tenfold, so the starts of the last pass
    // are then within about that much of the exact ones (float32 sums over a
    // segment differ by about 1e-5).  Segments whose start moved by less than
    // 4e-6 are not rerun.
    pp.tol = 4e-5f;
    pp.tol_skip = 4e-6f;
    pp.P = reinterpret_cast<float*>(ws + cl.off_pP);
    float* n_seg = reinterpret_cast<float*>(ws + cl.off_pn);
    // (Running the sums on the side stream beside the prep kernel gained
    // nothing: the prep kernel slowed by as much.)
    if ((e = vla::launch_state_prep(sp, a, nch, 0, nblk, 0, stream)) != hipSuccess) return hip_fail(e, "state prep launch");
    if ((e = vla::launch_para_init(pp, sp, pl.n_init, n_seg, stream)) != hipSuccess) return hip_fail(e, "para init launch");
    if ((e = vla::launch_para_sums(pp, sp, stream)) != hipSuccess) return hip_fail(e, "para sums launch");
    pp.iter_last = 0;
    if ((e = vla::launch_para_sweep(pp, 1, stream)) != hipSuccess) return hip_fail(e, "para sweep launch");
    vla::ChainSeg sg{};
    sg.pr = 1;
    sg.nseg = G;
    for (int sidx = 0; sidx <= G; ++sidx) sg.bnd[sidx] = pp.bnd[sidx];
    sg.S_in = pp.Sit;
    sg.n_in = n_seg;
    sg.F = reinterpret_cast<float*>(ws + cl.off_pF);
    sg.rec = reinterpret_cast<float*>(ws + cl.off_prec);
    sg.conv = pp.conv;
    sg.active = pp.active;
    const int passes = std::min(G, kParaPasses);
    for (int k = 0; k < passes; ++k) {
      hipEvent_t ev0, ev1;
      next_timing(&ev0, &ev1);
      if ((e = vla::launch_state_chain(sp, sg, a, pl.chain_info, nch, stream, ev0, ev1)) != hipSuccess)
        return hip_fail(e, "state chain launch");
      pp.iter_last = k + 1 == passes ? 1 : 0;
      if ((e = vla::launch_para_sweep(pp, 0, stream)) != hipSuccess) return hip_fail(e, "para sweep launch");
    }
    if ((e = vla::launch_para_stats(pp, a.S_T, a.n_T, stats, stream)) != hipSuccess) return hip_fail(e, "para stats launch");
    if ((e = vla::launch_state_readout(sp, a, pl.chain_info, nch, 0, nblk, 0, stream)) != hipSuccess)
      return hip_fail(e, "state readout launch");
  } else if (nseg == 1) {
    if ((e = vla::launch_state_prep(sp, a, nch, 0, nblk, 0, stream)) != hipSuccess) return hip_fail(e, "state prep launch");
    hipEvent_t ev0, ev1;
    next_timing(&ev0, &ev1);
    if ((e = vla::launch_state_chain(sp, chain_seg(0), a, pl.chain_info, nch, stream, ev0, ev1)) != hipSuccess)
      return hip_fail(e, "state chain launch");
    if ((e = vla::launch_state_readout(sp, a, pl.chain_info, nch, 0, nblk, 0, stream)) != hipSuccess)
      return hip_fail(e, "state readout launch");
  } else {
    std::lock_guard<std::mutex> lock(side_pool().mu);
    SideStream* ss = side_stream(&e);
    if (!ss) return hip_fail(e, "side stream setup");
    hipStream_t side = ss->stream;
    hipEvent_t ev_in = ss->ev[0], ev_end = ss->ev[1];
    hipEvent_t* ev_prep = ss->ev + 2;
    hipEvent_t* ev_chain = ss->ev + 2 + kMaxChainSegs;
    auto prep = [&](int sidx) {
      hipError_t r = vla::launch_state_prep(sp, a, nch, seg_lo(sidx), seg_lo(sidx + 1) - seg_lo(sidx),
                                 sidx == 0 ? 0 : ss->side_wg, side);
      return r != hipSuccess ? r : hipEventRecord(ev_prep[sidx], side);
    };
    if ((e = hipEventRecord(ev_in, stream)) != hipSuccess || (e = hipStreamWaitEvent(side, ev_in, 0)) != hipSuccess ||
        (e = prep(0)) != hipSuccess)
      return hip_fail(e, "state prep launch");
    for (int sidx = 0; sidx < nseg; ++sidx) {
      if (sidx + 1 < nseg && (e = prep(sidx + 1)) != hipSuccess) return hip_fail(e, "state prep launch");
      hipEvent_t ev0, ev1;
      next_timing(&ev0, &ev1);
      if ((e = hipStreamWaitEvent(stream, ev_prep[sidx], 0)) != hipSuccess ||
          (e = vla::launch_state_chain(sp, chain_seg(sidx), a, pl.chain_info, nch, stream, ev0, ev1)) != hipSuccess ||
          (e = hipEventRecord(ev_chain[sidx], stream)) != hipSuccess)
        return hip_fail(e, "state chain launch");
      if ((e = hipStreamWaitEvent(side, ev_chain[sidx], 0)) != hipSuccess ||
          (e = vla::launch_state_readout(sp, a, pl.chain_info, nch, seg_lo(sidx), seg_lo(sidx + 1) - seg_lo(sidx),
                                         sidx + 1 == nseg ? 0 : ss->side_wg, side)) != hipSuccess)
        return hip_fail(e, "state readout launch");
    }
    if ((e = hipEventRecord(ev_end, side)) != hipSuccess || (e = hipStreamWaitEvent(stream, ev_end, 0)) != hipSuccess)
      return hip_fail(e, "side stream join");
  }
  if ((e = vla::launch_stats_finalize(stats, pl.chain_info, static_cast<int>(chains), stream)) != hipSuccess)
    return hip_fail(e, "stats launch");
  e = vla::launch_scan_sequential(a, d, bf16, static_cast<int>(chains), pl.chain_info, stream);
  if (e != hipSuccess) return hip_fail(e, "chunked fallback launch");
  return VLA_OK;
}

namespace {
vla_status_t check_backward(const vla_scan_params_t* p) {
  vla_status_t s = check_params(p);
  if (s != VLA_OK) return s;
  if (p->d > 64) return fail(VLA_EUNSUPPORTED, "vla_scan_backward supports d = 16, 32, 64 (got %d)", p->d);
  if (p->update != VLA_UPDATE_ADDITIVE) return fail(VLA_EUNSUPPORTED, "vla_scan_backward supports the additive update");
  if (strided(p)) return fail(VLA_EUNSUPPORTED, "vla_scan_backward takes contiguous inputs (strides 0)");
  return VLA_OK;
}
}  // namespace

vla_status_t vla_scan_backward_workspace_size(const vla_scan_params_t* p, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(VLA_EINVAL, "bytes is NULL");
  const vla_status_t s = check_backward(p);
  if (s != VLA_OK) return s;
  *bytes = vla::bwd_workspace_bytes(static_cast<int64_t>(p->B) * p->H, p->T, p->d, p->r);
  return VLA_OK;
}

vla_status_t vla_scan_backward(const vla_scan_params_t* p, const void* q, const void* k, const void* v,
                               const void* u, const float* A0, const float* S0, const float* n0, const float* g_o,
                               const float* g_AT, const float* g_ST, const float* g_nT, float* g_q, float* g_k,
                               float* g_v, float* g_u, float* g_A0, float* g_S0, float* g_n0, void* workspace,
                               size_t workspace_bytes, void* stream_ptr) {
  g_last_error.clear();
  vla_status_t s = check_backward(p);
  if (s != VLA_OK) return s;
  const int64_t chains = static_cast<int64_t>(p->B) * p->H;
  if (chains == 0) return VLA_OK;
  const int d = p->d, r = p->r;
  const size_t es = dtype_size(p->in_dtype);
  const size_t n_tok = static_cast<size_t>(chains) * static_cast<size_t>(p->T);
  const size_t b_seq = n_tok * d * es, b_u = b_seq * r, b_g = n_tok * d * 4, b_gu = b_g * r;
  const size_t b_mat = static_cast<size_t>(chains) * d * d * 4, b_vec = static_cast<size_t>(chains) * d * 4;
  if (n_tok > 0 && (!q || !k || !v || !u || !g_o || !g_q || !g_k || !g_v || !g_u))
    return fail(VLA_EINVAL, "q, k, v, u, g_o and g_q, g_k, g_v, g_u must be non-NULL");
  if (!g_A0 || !g_S0 || !g_n0) return fail(VLA_EINVAL, "g_A0, g_S0 and g_n0 must be non-NULL");
  const void* al16[] = {q, k, v, u, g_o, g_q, g_k, g_v, g_u};
  for (const void* x : al16)
    if (n_tok > 0 && !aligned(x, 16)) return fail(VLA_EINVAL, "sequence tensors must be 16-byte aligned");
  const void* al4[] = {A0, S0, n0, g_AT, g_ST, g_nT, g_A0, g_S0, g_n0};
  for (const void* x : al4)
    if (!aligned(x, 4)) return fail(VLA_EINVAL, "state tensors must be 4-byte aligned");
  const struct { const void* p; size_t n; } ins[] = {{q, b_seq}, {k, b_seq}, {v, b_seq}, {u, b_u}, {A0, b_mat},
                                                     {S0, b_mat}, {n0, b_vec}, {g_o, b_g}, {g_AT, b_mat},
                                                     {g_ST, b_mat}, {g_nT, b_vec}};
  const struct { const void* p; size_t n; } outs[] = {{g_q, b_g}, {g_k, b_g}, {g_v, b_g}, {g_u, b_gu},
                                                      {g_A0, b_mat}, {g_S0, b_mat}, {g_n0, b_vec}};
  const int n_outs = static_cast<int>(sizeof(outs) / sizeof(outs[0]));
  for (int oi = 0; oi < n_outs; ++oi) {
    for (const auto& in : ins)
      if (overlap(outs[oi].p, outs[oi].n, in.p, in.n)) return fail(VLA_EINVAL, "a gradient overlaps an input");
    for (int oj = oi + 1; oj < n_outs; ++oj)
      if (overlap(outs[oi].p, outs[oi].n, outs[oj].p, outs[oj].n))
        return fail(VLA_EINVAL, "gradients overlap each other");
  }
  const size_t need = vla::bwd_workspace_bytes(chains, p->T, d, r);
  if (workspace_bytes < need || !workspace || !aligned(workspace, kAlign))
    return fail(VLA_EWORKSPACE, "workspace of %zu bytes (256-byte aligned) needed (got %zu)", need, workspace_bytes);
  for (const auto& in : ins)
    if (overlap(workspace, need, in.p, in.n)) return fail(VLA_EINVAL, "workspace overlaps an input");
  for (const auto& ot : outs)
    if (overlap(workspace, need, ot.p, ot.n)) return fail(VLA_EINVAL, "workspace overlaps a gradient");
  vla::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.u = u;
  a.A0 = A0; a.S0 = S0; a.n0 = n0;
  a.go = g_o; a.gAT = g_AT; a.gST = g_ST; a.gnT = g_nT;
  a.gq = g_q; a.gk = g_k; a.gv = g_v; a.gu = g_u; a.gA0 = g_A0; a.gS0 = g_S0; a.gn0 = g_n0;
  a.T = p->T; a.r = r; a.eps = p->eps;
  a.nudge_period = p->nudge_period;
  a.nudge_phase0 = p->nudge_period > 0 ? static_cast<int32_t>((p->t0 + 1) % p->nudge_period) : 0;
  a.cap_on = (p->s_cap > 0.f && std::isfinite(p->s_cap)) ? 1 : 0;
  a.cap = a.cap_on ? p->s_cap : 0.f;
  a.den_eps = p->den_eps;
  vla::bwd_carve(a, workspace, chains, p->T, d, r);
  const hipError_t e = vla::launch_backward(a, d, p->in_dtype == VLA_BF16, static_cast<int>(chains),
                                            static_cast<hipStream_t>(stream_ptr));
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return VLA_OK;
}

namespace {
// The fused entry point runs the prologue inside the two-wave sequential
// kernel when the call takes it (d <= 64, more than 16 tokens, sequential
// schedule); otherwise a prologue pass writes the features and u into the
// workspace first.
bool fused_in_kernel(const vla_scan_params_t* p) { return !plan_schedule(p).use && p->d <= 64 && p->T > 16; }

size_t fused_prologue_bytes(const vla_scan_params_t* p) {
  const size_t n = static_cast<size_t>(p->B) * p->H * p->T * p->d * dtype_size(p->in_dtype);
  return align_up(n) * 2 + align_up(n * p->r);
}

vla_status_t check_fused(const vla_scan_params_t* p) {
  const vla_status_t s = check_params(p);
  if (s != VLA_OK) return s;
  if (strided(p)) return fail(VLA_EUNSUPPORTED, "vla_scan_forward_fused takes contiguous inputs (strides 0)");
  if (p->validate) return fail(VLA_EUNSUPPORTED, "vla_scan_forward_fused has no validation pre-pass");
  return VLA_OK;
}
}  // namespace

vla_status_t vla_scan_fused_workspace_size(const vla_scan_params_t* p, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(VLA_EINVAL, "bytes is NULL");
  const vla_status_t s = check_fused(p);
  if (s != VLA_OK) return s;
  size_t need = 0;
  const vla_status_t s2 = vla_scan_workspace_size(p, &need);
  if (s2 != VLA_OK) return s2;
  *bytes = fused_in_kernel(p) ? need : fused_prologue_bytes(p) + need;
  return VLA_OK;
}

vla_status_t vla_scan_forward_fused(const vla_scan_params_t* p, const void* q_raw, const void* k_raw, const void* v,
                                    const void* W_u, const float* A0, const float* S0, const float* n0, void* o,
                                    float* A_T, float* S_T, float* n_T, int32_t* stats, void* workspace,
                                    size_t workspace_bytes, void* stream_ptr) {
  g_last_error.clear();
  vla_status_t s = check_fused(p);
  if (s != VLA_OK) return s;
  const int64_t chains = static_cast<int64_t>(p->B) * p->H;
  if (chains == 0) return VLA_OK;
  const int d = p->d, r = p->r;
  const size_t es = dtype_size(p->in_dtype);
  const size_t n_tok = static_cast<size_t>(chains) * static_cast<size_t>(p->T);
  const size_t b_seq = n_tok * d * es, b_w = static_cast<size_t>(r) * d * d * es;
  const size_t b_mat = static_cast<size_t>(chains) * d * d * 4, b_vec = static_cast<size_t>(chains) * d * 4;
  if (n_tok > 0 && (!q_raw || !k_raw || !v || !W_u || !o))
    return fail(VLA_EINVAL, "q_raw, k_raw, v, W_u and o must be non-NULL");
  if (!A_T || !S_T || !n_T) return fail(VLA_EINVAL, "A_T, S_T and n_T must be non-NULL");
  const void* seq[5] = {q_raw, k_raw, v, W_u, o};
  for (const void* x : seq)
    if (n_tok > 0 && !aligned(x, 16)) return fail(VLA_EINVAL, "q_raw, k_raw, v, W_u, o must be 16-byte aligned");
  if (!aligned(A0, 16) || !aligned(S0, 16) || !aligned(A_T, 16) || !aligned(S_T, 16) || !aligned(n0, 4) ||
      !aligned(n_T, 4))
    return fail(VLA_EINVAL, "state tensors misaligned (A, S: 16 bytes; n: 4 bytes)");
  const struct { const void* p; size_t n; } ins[] = {{q_raw, b_seq}, {k_raw, b_seq}, {v, b_seq}, {W_u, b_w}};
  const struct { const void* p; size_t n; const void* own; } outs[] = {
      {o, b_seq, nullptr}, {A_T, b_mat, A0}, {S_T, b_mat, S0}, {n_T, b_vec, n0},
      {stats, static_cast<size_t>(chains) * 16, nullptr}};
  const int n_outs = static_cast<int>(sizeof(outs) / sizeof(outs[0]));
  for (int oi = 0; oi < n_outs; ++oi) {
    const auto& ot = outs[oi];
    if (!ot.p) continue;
    for (const auto& in : ins)
      if (bad_alias(ot.p, ot.n, in.p, in.n, false)) return fail(VLA_EINVAL, "an output overlaps q_raw, k_raw, v or W_u");
    const struct { const void* p; size_t n; } st[] = {{A0, b_mat}, {S0, b_mat}, {n0, b_vec}};
    for (const auto& sx : st)
      if (bad_alias(ot.p, ot.n, sx.p, sx.n, ot.own == sx.p)) return fail(VLA_EINVAL, "outputs overlap the state");
    for (int oj = oi + 1; oj < n_outs; ++oj)
      if (overlap(ot.p, ot.n, outs[oj].p, outs[oj].n)) return fail(VLA_EINVAL, "outputs overlap each other");
  }
  size_t need = 0;
  if ((s = vla_scan_fused_workspace_size(p, &need)) != VLA_OK) return s;
  if (workspace_bytes < need || (need > 0 && (!workspace || !aligned(workspace, kAlign))))
    return fail(VLA_EWORKSPACE, "workspace of %zu bytes (256-byte aligned) needed (got %zu)", need, workspace_bytes);
  if (need > 0) {
    for (const auto& in : ins)
      if (overlap(workspace, need, in.p, in.n)) return fail(VLA_EINVAL, "workspace overlaps an input");
    for (const auto& ot : outs)
      if (overlap(workspace, need, ot.p, ot.n)) return fail(VLA_EINVAL, "workspace overlaps an output");
    const struct { const void* p; size_t n; } st[] = {{A0, b_mat}, {S0, b_mat}, {n0, b_vec}};
    for (const auto& sx : st)
      if (overlap(workspace, need, sx.p, sx.n)) return fail(VLA_EINVAL, "workspace overlaps the state");
  }
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const bool bf16 = p->in_dtype == VLA_BF16;
  if (!fused_in_kernel(p)) {
    // Prologue pass: q, k features and u into the workspace, then the scan.
    char* ws = static_cast<char*>(workspace);
    void* qf = ws;
    void* kf = ws + align_up(b_seq);
    void* uf = ws + 2 * align_up(b_seq);
    const size_t pro = fused_prologue_bytes(p);
    hipError_t e = vla::launch_feature_map(q_raw, k_raw, qf, kf, static_cast<int64_t>(n_tok) * d, bf16, stream);
    if (e == hipSuccess && n_tok > 0)
      e = vla::launch_project_u(static_cast<int64_t>(n_tok), d, r, bf16, bf16, W_u, k_raw, uf, stream);
    if (e != hipSuccess) return hip_fail(e, "fused prologue launch");
    return vla_scan_forward(p, qf, kf, v, uf, A0, S0, n0, o, A_T, S_T, n_T, stats,
                            need > pro ? ws + pro : nullptr, need - pro, stream_ptr);
  }
  vla::ScanArgs a{};
  a.q = q_raw; a.k = k_raw; a.v = v; a.u = nullptr;
  a.A0 = A0; a.S0 = S0; a.n0 = n0;
  a.o = o; a.A_T = A_T; a.S_T = S_T; a.n_T = n_T; a.stats = stats;
  a.T = p->T; a.r = r; a.eps = p->eps;
  a.nudge_period = p->nudge_period;
  a.nudge_phase0 = p->nudge_period > 0 ? static_cast<int32_t>((p->t0 + 1) % p->nudge_period) : 0;
  a.cap_on = (p->s_cap > 0.f && std::isfinite(p->s_cap)) ? 1 : 0;
  a.cap = a.cap_on ? p->s_cap : 0.f;
  a.den_eps = p->den_eps;
  a.residual = p->update == VLA_UPDATE_RESIDUAL ? 1 : 0;
  a.fused = 1;
  a.W_u = W_u;
  const hipError_t e = vla::launch_scan_split_fused(a, d, bf16, static_cast<int>(chains), stream);
  if (e != hipSuccess) return hip_fail(e, "fused scan launch");
  return VLA_OK;
}

vla_status_t vla_scan_forward_noalloc(const vla_scan_params_t* p, const void* q, const void* k, const void* v,
                                      const void* u, const float* A0, const float* S0, const float* n0, void* o,
                                      float* A_T, float* S_T, float* n_T, int32_t* stats, void* stream_ptr) {
  g_last_error.clear();
  size_t need = 0;
  vla_status_t s = vla_scan_workspace_size(p, &need);
  if (s != VLA_OK) return s;
  if (need > VLA_NOALLOC_SCRATCH_BYTES)
    return fail(VLA_EWORKSPACE,
                "this call needs %zu bytes of scratch; vla_scan_forward_noalloc holds %llu (use vla_scan_forward "
                "with a workspace)",
                need, static_cast<unsigned long long>(VLA_NOALLOC_SCRATCH_BYTES));
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "device query");
  if (dev < 0 || dev >= 64) return fail(VLA_EUNSUPPORTED, "device ordinal %d out of range", dev);
  void* ws = nullptr;
  {
    ScratchTable& tb = scratch_table();
    std::lock_guard<std::mutex> lock(tb.mu);
    if (!tb.ptr[dev]) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "scratch address lookup");
      if (!addr || !aligned(addr, kAlign)) return fail(VLA_EHIP, "scratch address lookup returned a bad address");
      tb.ptr[dev] = addr;
    }
    ws = tb.ptr[dev];
  }
  return vla_scan_forward(p, q, k, v, u, A0, S0, n0, o, A_T, S_T, n_T, stats, need > 0 ? ws : nullptr, need,
                          stream_ptr);
}

vla_status_t vla_scan_step(const vla_scan_params_t* p, const void* q, const void* k, const void* v, const void* u,
                           float* A, float* S, float* n, void* o, int32_t* stats, void* workspace,
                           size_t workspace_bytes, void* stream_ptr) {
  g_last_error.clear();
  if (!p) return fail(VLA_EINVAL, "params is NULL");
  if (p->T != 1) return fail(VLA_EINVAL, "vla_scan_step takes one token per chain (T = 1, got %d)", p->T);
  if (static_cast<int64_t>(p->B) * p->H > 0 && (!A || !S || !n))
    return fail(VLA_EINVAL, "A, S and n must be non-NULL (the state is updated in place)");
  return vla_scan_forward(p, q, k, v, u, A, S, n, o, A, S, n, stats, workspace, workspace_bytes, stream_ptr);
}

vla_status_t vla_project_u(int64_t rows, int32_t d, int32_t r, int32_t in_dtype, int32_t out_dtype,
                           const void* W_u, const void* k_raw, void* u, void* stream_ptr) {
  g_last_error.clear();
  if (rows < 0) return fail(VLA_EINVAL, "rows must be >= 0");
  if (!supported_d(d)) return fail(VLA_EUNSUPPORTED, "d = %d unsupported (16, 32, 64, 128)", d);
  if (r < 1 || r > 4) return fail(VLA_EUNSUPPORTED, "r = %d unsupported (1..4)", r);
  if ((in_dtype != VLA_F32 && in_dtype != VLA_BF16) || (out_dtype != VLA_F32 && out_dtype != VLA_BF16))
    return fail(VLA_EUNSUPPORTED, "dtype unsupported");
  if (rows == 0) return VLA_OK;
  if (!W_u || !k_raw || !u) return fail(VLA_EINVAL, "W_u, k_raw and u must be non-NULL");
  if (!aligned(W_u, 16) || !aligned(k_raw, 16) || !aligned(u, 16))
    return fail(VLA_EINVAL, "W_u, k_raw and u must be 16-byte aligned");
  const size_t b_in = dtype_size(in_dtype), b_out = dtype_size(out_dtype);
  if (overlap(u, static_cast<size_t>(rows) * r * d * b_out, k_raw, static_cast<size_t>(rows) * d * b_in) ||
      overlap(u, static_cast<size_t>(rows) * r * d * b_out, W_u, static_cast<size_t>(r) * d * d * b_in))
    return fail(VLA_EINVAL, "u overlaps its inputs");
  const hipError_t e = vla::launch_project_u(rows, d, r, in_dtype == VLA_BF16, out_dtype == VLA_BF16, W_u, k_raw,
                                             u, static_cast<hipStream_t>(stream_ptr));
  if (e != hipSuccess) return hip_fail(e, "projection launch");
  return VLA_OK;
}

const char* vla_status_string(vla_status_t s) {
  switch (s) {
    case VLA_OK: return "VLA_OK";
    case VLA_EINVAL: return "VLA_EINVAL";
    case VLA_EUNSUPPORTED: return "VLA_EUNSUPPORTED";
    case VLA_EWORKSPACE: return "VLA_EWORKSPACE";
    case VLA_ENONFINITE: return "VLA_ENONFINITE";
    case VLA_EHIP: return "VLA_EHIP";
  }
  return "VLA_UNKNOWN";
}

const char* vla_last_error(void) { return g_last_error.c_str(); }

vla_status_t vla_timing_enable(int32_t enable) {
  g_last_error.clear();
  Timing& tm = timing();
  std::lock_guard<std::mutex> lock(tm.mu);
  timing_release(tm);
  if (!enable) return VLA_OK;
  for (int i = 0; i < VLA_TIMING_SLOTS; ++i) {
    hipEvent_t a = nullptr, b = nullptr;
    // Timing only: no system-scope fence when they are recorded.
    hipError_t e = hipEventCreateWithFlags(&a, hipEventDisableSystemFence);
    if (e == hipSuccess) {
      e = hipEventCreateWithFlags(&b, hipEventDisableSystemFence);
      if (e != hipSuccess) (void)hipEventDestroy(a);
    }
    if (e != hipSuccess) {
      timing_release(tm);
      return hip_fail(e, "timing event creation");
    }
    tm.start.push_back(a);
    tm.stop.push_back(b);
  }
  tm.on = true;
  return VLA_OK;
}

vla_status_t vla_timing_collect(float* ms, int32_t cap, int32_t* n) {
  g_last_error.clear();
  if (!ms || !n || cap < 0) return fail(VLA_EINVAL, "vla_timing_collect: ms and n must be non-NULL, cap >= 0");
  Timing& tm = timing();
  std::lock_guard<std::mutex> lock(tm.mu);
  int written = 0;
  for (int i = 0; i < tm.used && written < cap; ++i) {
    hipError_t e = hipEventSynchronize(tm.stop[i]);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, tm.start[i], tm.stop[i]);
    if (e != hipSuccess) return hip_fail(e, "timing event readout");
    ms[written++] = t;
  }
  tm.used = 0;
  *n = written;
  return VLA_OK;
}

int vla_abi_version(void) { return VLA_ABI_VERSION; }

}  // extern "C"
