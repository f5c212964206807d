// C entry points of libselscan: argument checks, segmentation choice, launches.
// The operations are defined in include/selscan.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "selscan.h"
#include "sscan_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return SSCAN_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SSCAN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Compute units of the current device (cached per device); 256 if the query fails.
int device_cus() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (static_cast<int>(cache.size()) <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

struct SegPlan {
  int nseg;
  int64_t seg_len;
};

// The state entering every kBwdBlock-step block: [batch][ceil(L / kBwdBlock)][N][dim] fp32.
size_t checkpoint_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t N) {
  const int64_t nblk = (seqlen + sscan::kBwdBlock - 1) / sscan::kBwdBlock;
  return static_cast<size_t>(batch) * nblk * N * dim * sizeof(float);
}

size_t seg_workspace_bytes(int64_t batch, int64_t dim, int64_t N, int nseg) {
  if (nseg <= 1) return 0;
  // carry [nseg][B][D][N], end states [nseg][B][D][N], sums [nseg][B][D]
  return static_cast<size_t>(nseg) * batch * dim * (2 * N + 1) * sizeof(float);
}

// Segment count for a (batch, channel-tile) grid of `base` workgroups over `seqlen`
// steps, when `per_round` workgroups run at once (resident per CU x CUs).  One
// segment if the grid alone fills a round.  Otherwise the count, between the one
// that gives two rounds of workgroups and four times that (and with segments of at
// least min_len steps), whose last round is fullest: a grid just past a multiple of
// the round leaves a nearly empty last round, measured at up to 30 % slower.
int64_t pick_segments(int64_t base, int64_t seqlen, int64_t per_round, int64_t min_len) {
  if (base <= 0 || base >= per_round) return 1;
  const int64_t lo = (2 * per_round + base - 1) / base;
  int64_t hi = 4 * lo;
  const int64_t cap = seqlen / min_len < 1024 ? seqlen / min_len : 1024;
  if (hi > cap) hi = cap;
  if (lo > hi) return hi < 1 ? 1 : hi;
  int64_t best = lo;
  double best_fill = -1.0;
  for (int64_t n = lo; n <= hi; ++n) {
    const int64_t wgs = base * n;
    const int64_t rounds = (wgs + per_round - 1) / per_round;
    const double fill = static_cast<double>(wgs) / static_cast<double>(rounds * per_round);
    if (fill > best_fill + 1e-9) {
      best_fill = fill;
      best = n;
    }
  }
  return best;
}

// Segment count of a split output-mode forward by a cost model: the passes run in
// rounds of per_round workgroups (two per CU), each round as long as a segment plus
// a fixed pipeline fill and drain of two chunks; a last round at most half full costs
// 0.6 of a round (its workgroups have a CU each, and run faster).  Candidates run from
// the count that fills 90 % of one round to eight times that, with segments of at
// least four chunks, and segment lengths rounded up to whole chunks as the plan does;
// on equal costs the fewest segments win.  The 0.6 was fitted to a sweep of 15 split
// shapes (fp32 and bf16, 24 to 128 (batch, tile) workgroups, 1K to 128K steps), over
// which the pick was the fastest count or within 4 % of it; the mamba130m layer
// (batch 2, 2048 steps, dim 1536) gets 10 segments, 0.083 ms, where a rule that only
// maximised the last round's fill took 16, 0.087 ms.
int64_t pick_segments_out(int64_t base, int64_t seqlen, int64_t per_round) {
  if (base <= 0 || base >= per_round / 2) return 1;
  constexpr int64_t T = sscan::kChunk;
  int64_t lo = (9 * per_round + 10 * base - 1) / (10 * base);
  int64_t hi = 8 * lo;
  const int64_t cap = seqlen / (4 * T) < 1024 ? seqlen / (4 * T) : 1024;
  if (hi > cap) hi = cap;
  if (lo > hi) lo = 1;
  int64_t best = 1;
  double best_cost = -1.0;
  for (int64_t want = lo; want <= hi; ++want) {
    int64_t len = (seqlen + want - 1) / want;
    len = (len + T - 1) / T * T;
    const int64_t nseg = (seqlen + len - 1) / len;
    const int64_t wgs = base * nseg;
    const int64_t full = wgs / per_round, rem = wgs % per_round;
    const double rounds = static_cast<double>(full) + (rem == 0 ? 0.0 : (2 * rem <= per_round ? 0.6 : 1.0));
    const double cost = rounds * static_cast<double>(len + 2 * T);
    if (best_cost < 0.0 || cost < best_cost) {
      best_cost = cost;
      best = nseg;
    }
  }
  return best;
}

// Segments of the forward.  A grid of at least one workgroup per CU runs unsplit.  A
// smaller one is split, and its main pass then runs two states per wave, whose LDS use
// lets two workgroups share a CU, so the split aims at rounds of 2 x CUs workgroups
// (pick_segments_out).  The checkpoint pass of the backward keeps one state per wave
// and one-per-CU rounds.
int auto_segments(int64_t batch, int64_t seqlen, int64_t dim, int mode) {
  const int64_t base = (dim + sscan::kTile - 1) / sscan::kTile * batch;
  const int64_t cus = device_cus();
  if (base >= cus) return 1;
  if (mode == sscan::kFwdOut) return static_cast<int>(pick_segments_out(base, seqlen, 2 * cus));
  return static_cast<int>(pick_segments(base, seqlen, cus, 4 * sscan::kChunk));
}

// States per wave of a forward launch of nwg workgroups: two once there are more
// workgroups than CUs (so a CU can hold two), one otherwise.  Measured on the
// 256-workgroup training shape: one state per wave 0.476 ms, two 0.556 ms; on split
// shapes two states per wave won (long context 3.45 -> 2.69 ms).
int fwd_states_per_wave(int64_t N, int64_t nwg) { return (N >= 3 && nwg > device_cus()) ? 2 : 1; }

SegPlan plan_segments(int64_t batch, int64_t seqlen, int64_t dim, int64_t N, int64_t requested,
                      size_t ws_bytes, bool have_ws, int mode = sscan::kFwdOut) {
  int64_t want = requested > 0 ? requested : auto_segments(batch, seqlen, dim, mode);
  const int64_t maxseg = (seqlen + sscan::kChunk - 1) / sscan::kChunk;
  if (want > maxseg) want = maxseg;
  if (want < 1) want = 1;
  while (want > 1 && (!have_ws || seg_workspace_bytes(batch, dim, N, static_cast<int>(want)) > ws_bytes)) --want;
  SegPlan pl{1, seqlen};
  if (want <= 1) return pl;
  int64_t len = (seqlen + want - 1) / want;
  len = (len + sscan::kChunk - 1) / sscan::kChunk * sscan::kChunk;
  pl.seg_len = len;
  pl.nseg = static_cast<int>((seqlen + len - 1) / len);
  return pl;
}

bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes) {
  if (!a || !b || abytes == 0 || bbytes == 0) return false;
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return pa < pb + bbytes && pb < pa + abytes;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Buf {
  const void* p;
  size_t n;
};

int check_common(int64_t batch, int64_t dim, int64_t dstate, int dtype, unsigned flags) {
  if (dtype != SSCAN_F32 && dtype != SSCAN_BF16) return fail(SSCAN_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (flags & ~(SSCAN_FLAG_EULER | SSCAN_FLAG_STRUCTURED_A))
    return fail(SSCAN_ERR_UNSUPPORTED, "unknown flag bits 0x%x", flags);
  if (dstate < 1 || dstate > SSCAN_MAX_DSTATE)
    return fail(SSCAN_ERR_UNSUPPORTED, "dstate %lld outside [1, %d]", (long long)dstate, SSCAN_MAX_DSTATE);
  if (batch < 0 || dim < 0) return fail(SSCAN_ERR_INVALID_ARG, "negative size (batch %lld, dim %lld)",
                                        (long long)batch, (long long)dim);
  return SSCAN_OK;
}

// Convolution prologue arguments (all null / 0 for the plain scan).
struct ConvArgs {
  int64_t dconv;
  const float* w;
  const float* b;
  const float* state_in;
  float* state_out;
};

int check_conv(const ConvArgs& cv, int64_t batch, int64_t dim) {
  if (!cv.w) return SSCAN_OK;
  if (cv.dconv < 1 || cv.dconv > sscan::kMaxConv)
    return fail(SSCAN_ERR_UNSUPPORTED, "dconv %lld outside [1, %d]", (long long)cv.dconv, sscan::kMaxConv);
  if (!aligned(cv.w, 4) || (cv.b && !aligned(cv.b, 4)) || (cv.state_in && !aligned(cv.state_in, 4)) ||
      (cv.state_out && !aligned(cv.state_out, 4)))
    return fail(SSCAN_ERR_INVALID_ARG, "float32 tensor not 4-byte aligned");
  const size_t cs = static_cast<size_t>(batch) * dim * (cv.dconv - 1) * 4;
  if (cv.state_in && cv.state_out && cv.state_in != cv.state_out && overlaps(cv.state_in, cs, cv.state_out, cs))
    return fail(SSCAN_ERR_INVALID_ARG, "conv_state_in and conv_state_out partially overlap");
  return SSCAN_OK;
}

// Scratch of sscan_fwd_noalloc: the split forward's carries, segment end states and
// step sums, in a static device array instead of a caller's workspace.  Each device
// the library runs on holds one copy until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: kernels and copies get the address
// that hipGetSymbolAddress reports for the current device (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[SSCAN_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up once per device (with
// that device current) and cached; nullptr and an error message on failure.
void* noalloc_scratch(int* rc) {
  static std::mutex mu;
  static std::vector<void*> ptrs;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    *rc = hip_fail(e != hipSuccess ? e : hipErrorInvalidDevice, "hipGetDevice");
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(mu);
  if (static_cast<int>(ptrs.size()) <= dev) ptrs.resize(dev + 1, nullptr);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *rc = hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
      return nullptr;
    }
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

int fwd_impl(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype, unsigned flags, const void* x,
             const void* delta, const float* A, const void* B, const void* C, const float* D, const void* z,
             const float* delta_bias, const float* initial_state, void* y, float* last_state, void* workspace,
             size_t workspace_bytes, int64_t num_segments, void* stream, const ConvArgs& cv,
             float* ckpt_out = nullptr, size_t ckpt_bytes = 0) {
  int rc = check_common(batch, dim, dstate, dtype, flags);
  if (rc) return rc;
  rc = check_conv(cv, batch, dim);
  if (rc) return rc;
  if (seqlen < 0) return fail(SSCAN_ERR_INVALID_ARG, "negative seqlen %lld", (long long)seqlen);
  if (seqlen > SSCAN_MAX_SEQLEN)
    return fail(SSCAN_ERR_INVALID_ARG, "seqlen %lld above SSCAN_MAX_SEQLEN (%lld)", (long long)seqlen,
                (long long)SSCAN_MAX_SEQLEN);
  if (num_segments < 0) return fail(SSCAN_ERR_INVALID_ARG, "negative num_segments");
  const int64_t max_elems = (int64_t(1) << 62) / 8;
  if (batch > 0 && dim > 0 && seqlen > max_elems / batch / dim)
    return fail(SSCAN_ERR_INVALID_ARG, "batch*seqlen*dim too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t N = dstate;
  const size_t es = dtype == SSCAN_BF16 ? 2 : 4;
  const size_t tok = static_cast<size_t>(batch) * seqlen * dim * es;
  const size_t bc = static_cast<size_t>(batch) * seqlen * N * es;
  const size_t st = static_cast<size_t>(batch) * dim * N * sizeof(float);
  if (batch == 0 || dim == 0) return ok();
  const size_t conv_bytes = cv.w ? static_cast<size_t>(batch) * dim * (cv.dconv - 1) * 4 : 0;

  if (seqlen == 0) {
    if (cv.w && cv.state_out && cv.state_out != cv.state_in) {
      hipError_t e = sscan::launch_conv_state(x, cv.state_in, cv.state_out, batch, 0, dim, static_cast<int>(cv.dconv),
                                              dtype == SSCAN_BF16, s);
      if (e != hipSuccess) return hip_fail(e, "conv state launch");
    }
    if (last_state) {
      if (initial_state && !aligned(initial_state, 4)) return fail(SSCAN_ERR_INVALID_ARG, "initial_state misaligned");
      if (!aligned(last_state, 4)) return fail(SSCAN_ERR_INVALID_ARG, "last_state misaligned");
      if (initial_state != last_state) {
        if (overlaps(initial_state, st, last_state, st))
          return fail(SSCAN_ERR_INVALID_ARG, "initial_state and last_state partially overlap");
        hipError_t e = sscan::launch_fill_state(last_state, initial_state, batch * dim * N, s);
        if (e != hipSuccess) return hip_fail(e, "fill_state launch");
      }
    }
    return ok();
  }

  if (!x || !delta || !A || !B || !C || !y)
    return fail(SSCAN_ERR_INVALID_ARG, "null required pointer (x, delta, A, B, C and y are required)");
  if (!aligned(x, es) || !aligned(delta, es) || !aligned(y, es) || (z && !aligned(z, es)) || !aligned(B, es) ||
      !aligned(C, es))
    return fail(SSCAN_ERR_INVALID_ARG, "token tensor not aligned to its element size");
  if (!aligned(A, 4) || (D && !aligned(D, 4)) || (delta_bias && !aligned(delta_bias, 4)) ||
      (initial_state && !aligned(initial_state, 4)) || (last_state && !aligned(last_state, 4)) ||
      (workspace && !aligned(workspace, 4)))
    return fail(SSCAN_ERR_INVALID_ARG, "float32 tensor not 4-byte aligned");
  if (overlaps(y, tok, x, tok) || overlaps(y, tok, delta, tok) || overlaps(y, tok, z, tok) || overlaps(y, tok, B, bc) ||
      overlaps(y, tok, C, bc) || overlaps(y, tok, A, N * dim * 4))
    return fail(SSCAN_ERR_INVALID_ARG, "y overlaps an input");
  if (last_state) {
    if (overlaps(last_state, st, y, tok) || overlaps(last_state, st, x, tok) || overlaps(last_state, st, delta, tok) ||
        overlaps(last_state, st, z, tok) || overlaps(last_state, st, B, bc) || overlaps(last_state, st, C, bc))
      return fail(SSCAN_ERR_INVALID_ARG, "last_state overlaps y or an input");
    if (initial_state && initial_state != last_state && overlaps(initial_state, st, last_state, st))
      return fail(SSCAN_ERR_INVALID_ARG, "initial_state and last_state partially overlap");
  }
  const int64_t nblk = (seqlen + sscan::kBwdBlock - 1) / sscan::kBwdBlock;
  if (ckpt_out) {
    const size_t need = checkpoint_bytes(batch, seqlen, dim, N);
    if (!aligned(ckpt_out, 4)) return fail(SSCAN_ERR_INVALID_ARG, "checkpoints not 4-byte aligned");
    if (ckpt_bytes < need)
      return fail(SSCAN_ERR_INVALID_ARG, "checkpoint buffer too small (%zu < %zu bytes)", ckpt_bytes, need);
    const Buf others[] = {{x, tok}, {delta, tok}, {z, tok}, {y, tok}, {B, bc}, {C, bc}, {last_state, st},
                          {initial_state, st}, {A, static_cast<size_t>(N) * dim * 4}, {workspace, workspace_bytes}};
    for (const Buf& o : others)
      if (overlaps(ckpt_out, need, o.p, o.n)) return fail(SSCAN_ERR_INVALID_ARG, "checkpoints overlap a tensor");
  }
  if (cv.state_out) {
    const Buf others[] = {{x, tok}, {delta, tok}, {z, tok}, {y, tok}, {B, bc}, {C, bc}, {last_state, st},
                          {initial_state, st}, {cv.w, static_cast<size_t>(dim) * cv.dconv * 4}};
    for (const Buf& o : others)
      if (overlaps(cv.state_out, conv_bytes, o.p, o.n)) return fail(SSCAN_ERR_INVALID_ARG, "conv_state_out overlaps a tensor");
  }

  const SegPlan pl = plan_segments(batch, seqlen, dim, N, num_segments, workspace_bytes, workspace != nullptr);
  if (pl.nseg > 1) {
    // the split writes its aggregates and carries into the workspace before the main
    // pass reads the inputs, so the used part may overlap no tensor of the call
    const size_t used = seg_workspace_bytes(batch, dim, N, pl.nseg);
    const Buf others[] = {{x, tok}, {delta, tok}, {z, tok}, {y, tok}, {B, bc}, {C, bc},
                          {A, static_cast<size_t>(N) * dim * 4}, {D, static_cast<size_t>(dim) * 4},
                          {delta_bias, static_cast<size_t>(dim) * 4}, {initial_state, st}, {last_state, st},
                          {cv.w, cv.w ? static_cast<size_t>(dim) * cv.dconv * 4 : 0},
                          {cv.b, cv.b ? static_cast<size_t>(dim) * 4 : 0}, {cv.state_in, conv_bytes},
                          {cv.state_out, conv_bytes}};
    for (const Buf& o : others)
      if (overlaps(workspace, used, o.p, o.n)) return fail(SSCAN_ERR_INVALID_ARG, "workspace overlaps a tensor");
  }

  sscan::FwdParams p{};
  p.x = x; p.dt = delta; p.z = z; p.B = B; p.C = C;
  p.A = A; p.Dskip = D; p.bias = delta_bias;
  p.y = y; p.h_last = last_state;
  p.batch = batch; p.L = seqlen; p.dim = dim; p.N = static_cast<int>(N);
  p.ndtiles = (dim + sscan::kTile - 1) / sscan::kTile;
  p.seg_len = pl.seg_len; p.nseg = pl.nseg;
  p.npw = fwd_states_per_wave(N, p.ndtiles * batch * pl.nseg);
  p.euler = (flags & SSCAN_FLAG_EULER) != 0;
  p.structured = (flags & SSCAN_FLAG_STRUCTURED_A) != 0;
  p.conv_w = cv.w; p.conv_b = cv.b; p.conv_s = cv.state_in; p.dconv = static_cast<int>(cv.w ? cv.dconv : 0);
  p.ckpt = ckpt_out; p.nblk = nblk;
  const bool bf16 = dtype == SSCAN_BF16;
  // the convolution state leaves after the scan (which reads the incoming one)
  auto finish = [&]() -> int {
    if (cv.w && cv.state_out) {
      hipError_t e = sscan::launch_conv_state(x, cv.state_in, cv.state_out, batch, seqlen, dim,
                                              static_cast<int>(cv.dconv), bf16, s);
      if (e != hipSuccess) return hip_fail(e, "conv state launch");
    }
    return ok();
  };

  if (pl.nseg == 1) {
    p.h_init = initial_state;
    hipError_t e = sscan::launch_fwd_main(p, bf16, s);
    if (e != hipSuccess) return hip_fail(e, "scan launch");
    return finish();
  }

  const int64_t bdn = batch * dim * N;
  float* ws = static_cast<float*>(workspace);
  float* carry = ws;
  float* agg_h = ws + pl.nseg * bdn;
  float* agg_s = ws + 2 * pl.nseg * bdn;
  p.agg_h = agg_h;
  p.agg_s = agg_s;
  hipError_t e = sscan::launch_fwd_aggregate(p, bf16, s);
  if (e != hipSuccess) return hip_fail(e, "segment aggregate launch");
  e = sscan::launch_fwd_carry(agg_h, agg_s, A, initial_state, carry, batch, dim, static_cast<int>(N), pl.nseg, s);
  if (e != hipSuccess) return hip_fail(e, "segment carry launch");
  p.h_init = carry;
  e = sscan::launch_fwd_main(p, bf16, s);
  if (e != hipSuccess) return hip_fail(e, "scan launch");
  return finish();
}


// ---------------------------------------------------------------------------
// Backward pass: workspace layout and host checks.
// ---------------------------------------------------------------------------
size_t round256(size_t v) { return (v + 255) & ~size_t(255); }

struct BwdLayout {
  size_t ckpt, gB, gC, gA, gD, gb, seg, rg, rs, gin, total;
  size_t total_saved;      // bytes needed when the checkpoints come from the caller
  int nseg;                // forward (checkpoint) pass segments
  int64_t seg_len;
  int bseg;                // reverse pass segments
  int64_t seg_blocks;      // kBwdBlock-step blocks per reverse segment
  bool shared;             // the two passes share their segments (below)
};

// Reverse-pass segments: two reverse-kernel workgroups are resident per CU (LDS).  A
// smaller grid takes the forward's round cost model (pick_segments_out): on the
// mamba130m layer it picks 10 segments, sscan_bwd 0.264 ms, where the fill-only rule's
// 32 took 0.270 (16: 0.261; long context: 64 either way, 9.47 ms).
int bwd_segments(int64_t batch, int64_t seqlen, int64_t dim) {
  const int64_t ndt = (dim + sscan::kTile - 1) / sscan::kTile;
  const int64_t base = ndt * batch;
  const int64_t cus = device_cus();
  if (base <= 0) return 1;
  if (base >= cus) return base >= 2 * cus ? 1 : 2;   // two segments fill the second slot per CU
  return static_cast<int>(pick_segments_out(base, seqlen, 2 * cus));
}

// Segments of the two passes.  When the checkpoint pass is itself split (a grid of
// fewer workgroups than CUs) and N == 16, it takes the reverse pass's segment count
// and the reverse pass takes its segments: then every checkpoint workgroup also forms
// its segment's reverse aggregate (the kFwdCkptAgg mode with per-segment aggregates),
// and the reverse pass skips its aggregate sweep.  The checkpoint pass runs one
// workgroup per CU, so its length is its rounds times L/S steps either way: the long
// context's 64 segments take the same 10 x 2048 steps as its own plan's 32 (5 x 4096),
// the mamba130m layer's 10 take 2 x 208 against 3 x 128.  Measured, the aggregate
// sweep it saves is worth far more (long context sscan_bwd 9.58 -> 8.97 ms).
BwdLayout bwd_layout(int64_t batch, int64_t seqlen, int64_t dim, int64_t N) {
  BwdLayout lo{};
  const int64_t nblk = (seqlen + sscan::kBwdBlock - 1) / sscan::kBwdBlock;
  const int64_t ndt = (dim + sscan::kTile - 1) / sscan::kTile;
  const int want = bwd_segments(batch, seqlen, dim);
  lo.seg_blocks = (nblk + want - 1) / want;
  if (lo.seg_blocks < 1) lo.seg_blocks = 1;
  lo.bseg = static_cast<int>((nblk + lo.seg_blocks - 1) / lo.seg_blocks);
  if (lo.bseg < 1) lo.bseg = 1;
  SegPlan pl = plan_segments(batch, seqlen, dim, N, 0, ~size_t(0), true, sscan::kFwdCkpt);
  lo.shared = false;
  if (N == 16 && pl.nseg > 1 && lo.bseg > 1) {
    const SegPlan ps = plan_segments(batch, seqlen, dim, N, lo.bseg, ~size_t(0), true, sscan::kFwdCkpt);
    const int64_t sb = ps.seg_len / sscan::kBwdBlock;
    if (ps.nseg > 1 && ps.seg_len % sscan::kChunk == 0 && (nblk + sb - 1) / sb == ps.nseg) {
      pl = ps;
      lo.seg_blocks = sb;
      lo.bseg = ps.nseg;
      lo.shared = true;
    }
  }
  const size_t bdn = static_cast<size_t>(batch) * dim * N;
  size_t off = 0;
  lo.gB = off;   off += round256(static_cast<size_t>(ndt) * batch * N * seqlen * 4);
  lo.gC = off;   off += round256(static_cast<size_t>(ndt) * batch * N * seqlen * 4);
  lo.gA = off;   off += round256(static_cast<size_t>(lo.bseg) * bdn * 4);
  lo.gD = off;   off += round256(static_cast<size_t>(lo.bseg) * batch * dim * 4);
  lo.gb = off;   off += round256(static_cast<size_t>(lo.bseg) * batch * dim * 4);
  lo.nseg = pl.nseg;
  lo.seg_len = pl.seg_len;
  lo.seg = off;  off += round256(seg_workspace_bytes(batch, dim, N, pl.nseg));
  const size_t nb = lo.bseg > 1 ? static_cast<size_t>(lo.bseg) : 0;
  lo.rg = off;   off += round256(nb * bdn * 4);
  lo.rs = off;   off += round256(nb * batch * dim * 4);
  lo.gin = off;  off += round256(nb * bdn * 4);
  lo.total_saved = off;
  // the checkpoints come last, so a caller that supplies its own can pass less
  lo.ckpt = off; off += round256(checkpoint_bytes(batch, seqlen, dim, N));
  lo.total = off;
  return lo;
}

int bwd_impl(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype, unsigned flags, const void* x,
             const void* delta, const float* A, const void* B, const void* C, const float* D, const void* z,
             const float* delta_bias, const float* initial_state, const void* dy, const float* dlast_state,
             void* dx, void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz, float* ddelta_bias,
             float* dinitial_state, void* workspace, size_t workspace_bytes, void* stream,
             const float* ckpt_in = nullptr, size_t ckpt_bytes = 0, bool saved = false) {
  int rc = check_common(batch, dim, dstate, dtype, flags);
  if (rc) return rc;
  if (seqlen < 0) return fail(SSCAN_ERR_INVALID_ARG, "negative seqlen %lld", (long long)seqlen);
  if (seqlen > SSCAN_MAX_SEQLEN)
    return fail(SSCAN_ERR_INVALID_ARG, "seqlen %lld above SSCAN_MAX_SEQLEN (%lld)", (long long)seqlen,
                (long long)SSCAN_MAX_SEQLEN);
  const int64_t max_elems = (int64_t(1) << 62) / 8;
  if (batch > 0 && dim > 0 && seqlen > max_elems / batch / dim)
    return fail(SSCAN_ERR_INVALID_ARG, "batch*seqlen*dim too large");
  if (saved && seqlen > 0 && batch > 0 && dim > 0 && !ckpt_in)
    return fail(SSCAN_ERR_INVALID_ARG, "null required pointer (checkpoints)");
  if ((z == nullptr) != (dz == nullptr)) return fail(SSCAN_ERR_INVALID_ARG, "dz must be given exactly when z is");
  if (dD && !D) return fail(SSCAN_ERR_INVALID_ARG, "dD requested without D");
  if (dim > (int64_t(1) << 27)) return fail(SSCAN_ERR_INVALID_ARG, "dim too large for the backward pass");
  const int64_t N = dstate;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (batch == 0 || dim == 0) return ok();
  if (!dA) return fail(SSCAN_ERR_INVALID_ARG, "null required pointer (dA)");
  const size_t es = dtype == SSCAN_BF16 ? 2 : 4;
  if (seqlen == 0) {
    // no steps: every gradient is zero except dh0 = dLoss/d(last state)
    hipError_t e = sscan::launch_fill_state(dA, nullptr, dim * N, s);
    if (e == hipSuccess && dD) e = sscan::launch_fill_state(dD, nullptr, dim, s);
    if (e == hipSuccess && ddelta_bias) e = sscan::launch_fill_state(ddelta_bias, nullptr, dim, s);
    if (e == hipSuccess && dinitial_state) e = sscan::launch_fill_state(dinitial_state, dlast_state, batch * dim * N, s);
    if (e != hipSuccess) return hip_fail(e, "fill launch");
    return ok();
  }
  if (!x || !delta || !A || !B || !C || !dy || !dx || !ddelta || !dB || !dC)
    return fail(SSCAN_ERR_INVALID_ARG,
                "null required pointer (x, delta, A, B, C, dy, dx, ddelta, dA, dB and dC are required)");
  const void* tok_ptrs[] = {x, delta, z, dy, dx, ddelta, dz, B, C, dB, dC};
  for (const void* q : tok_ptrs)
    if (q && !aligned(q, es)) return fail(SSCAN_ERR_INVALID_ARG, "token tensor not aligned to its element size");
  const void* f32_ptrs[] = {A, D, delta_bias, initial_state, dlast_state, dA, dD, ddelta_bias, dinitial_state};
  for (const void* q : f32_ptrs)
    if (q && !aligned(q, 4)) return fail(SSCAN_ERR_INVALID_ARG, "float32 tensor not 4-byte aligned");
  if (!workspace || !aligned(workspace, 256))
    return fail(SSCAN_ERR_INVALID_ARG, "workspace missing or not 256-byte aligned");
  const BwdLayout lo = bwd_layout(batch, seqlen, dim, N);
  const size_t ws_need = saved ? lo.total_saved : lo.total;
  if (workspace_bytes < ws_need)
    return fail(SSCAN_ERR_INVALID_ARG, "workspace too small (%zu < %zu bytes)", workspace_bytes, ws_need);
  if (saved) {
    const size_t need = checkpoint_bytes(batch, seqlen, dim, N);
    if (!aligned(ckpt_in, 4)) return fail(SSCAN_ERR_INVALID_ARG, "checkpoints not 4-byte aligned");
    if (ckpt_bytes < need)
      return fail(SSCAN_ERR_INVALID_ARG, "checkpoint buffer too small (%zu < %zu bytes)", ckpt_bytes, need);
  }

  const size_t tok = static_cast<size_t>(batch) * seqlen * dim * es;
  const size_t bc = static_cast<size_t>(batch) * seqlen * N * es;
  const size_t st = static_cast<size_t>(batch) * dim * N * 4;
  const Buf inputs[] = {{x, tok}, {delta, tok}, {z, tok}, {dy, tok}, {B, bc}, {C, bc}, {A, size_t(dim) * N * 4},
                        {D, size_t(dim) * 4}, {delta_bias, size_t(dim) * 4}, {initial_state, st},
                        {dlast_state, st}};
  const size_t ckn = saved ? checkpoint_bytes(batch, seqlen, dim, N) : 0;
  const Buf inputs2[] = {{ckpt_in, ckn}};
  const Buf outputs[] = {{dx, tok}, {ddelta, tok}, {dz, tok}, {dB, bc}, {dC, bc}, {dA, size_t(dim) * N * 4},
                         {dD, size_t(dim) * 4}, {ddelta_bias, size_t(dim) * 4}, {dinitial_state, st},
                         {workspace, ws_need}};
  for (const Buf& o : outputs)
    for (const Buf& i : inputs2)
      if (overlaps(o.p, o.n, i.p, i.n)) return fail(SSCAN_ERR_INVALID_ARG, "an output overlaps the checkpoints");
  for (const Buf& o : outputs) {
    for (const Buf& i : inputs)
      if (overlaps(o.p, o.n, i.p, i.n)) return fail(SSCAN_ERR_INVALID_ARG, "an output overlaps an input");
    for (const Buf& o2 : outputs)
      if (&o2 != &o && overlaps(o.p, o.n, o2.p, o2.n)) return fail(SSCAN_ERR_INVALID_ARG, "outputs overlap");
  }

  char* ws = static_cast<char*>(workspace);
  const bool bf16 = dtype == SSCAN_BF16;
  const bool euler = (flags & SSCAN_FLAG_EULER) != 0;
  const int64_t nblk = (seqlen + sscan::kBwdBlock - 1) / sscan::kBwdBlock;
  const int64_t ndt = (dim + sscan::kTile - 1) / sscan::kTile;
  const float* ckpt = saved ? ckpt_in : reinterpret_cast<const float*>(ws + lo.ckpt);
  // The checkpoint pass also forms the reverse pass's segment carries when it runs as
  // one sweep over the sequence and the reverse pass has two segments (the count
  // bwd_segments gives for one to two workgroups per CU), N == 16, the second starting
  // at a chunk start: the sweep already forms every Abar, and the separate aggregate
  // sweep and carry kernel are skipped.
  const int64_t rseg_len = lo.seg_blocks * sscan::kBwdBlock;
  const bool agg_in_ckpt = !saved && lo.nseg == 1 && N == 16 && lo.bseg == 2 && rseg_len % sscan::kChunk == 0;
  // a split checkpoint pass whose segments the reverse pass shares forms the reverse
  // aggregates of every segment (bwd_layout)
  const bool seg_agg = !saved && lo.shared;
  hipError_t e;
  if (!saved) {
  // 1. checkpoints: the forward recurrence, storing the state entering every chunk
  sscan::FwdParams p{};
  p.x = x; p.dt = delta; p.z = nullptr; p.B = B; p.C = C;
  p.A = A; p.Dskip = nullptr; p.bias = delta_bias;
  p.y = nullptr; p.h_last = nullptr;
  p.batch = batch; p.L = seqlen; p.dim = dim; p.N = static_cast<int>(N);
  p.ndtiles = ndt; p.nblk = nblk;
  p.seg_len = lo.seg_len; p.nseg = lo.nseg;
  p.npw = 1;
  p.euler = euler;
  p.ckpt = reinterpret_cast<float*>(ws + lo.ckpt);
  if (lo.nseg == 1) {
    p.h_init = initial_state;
  } else {
    const int64_t bdn = batch * dim * N;
    float* sw = reinterpret_cast<float*>(ws + lo.seg);
    float* carry = sw;
    p.agg_h = sw + lo.nseg * bdn;
    p.agg_s = sw + 2 * lo.nseg * bdn;
    // the aggregate pass with two states per wave (two workgroups share a CU); the
    // checkpoint pass itself runs the row layout
    p.npw = N >= 3 ? 2 : 1;
    e = sscan::launch_fwd_aggregate(p, bf16, s);
    p.npw = 1;
    if (e != hipSuccess) return hip_fail(e, "segment aggregate launch");
    e = sscan::launch_fwd_carry(p.agg_h, p.agg_s, A, initial_state, carry, batch, dim, static_cast<int>(N),
                                lo.nseg, s);
    if (e != hipSuccess) return hip_fail(e, "segment carry launch");
    p.h_init = carry;
  }
  if (agg_in_ckpt) {
    p.z = z;
    p.dy = dy;
    p.dlast = dlast_state;
    p.gin = reinterpret_cast<float*>(ws + lo.gin);
    p.rseg_len = rseg_len;
    e = sscan::launch_fwd_checkpoints_agg(p, bf16, s);
  } else if (seg_agg) {
    p.z = z;
    p.dy = dy;
    p.gin = reinterpret_cast<float*>(ws + lo.rg);
    p.ragg_s = reinterpret_cast<float*>(ws + lo.rs);
    p.rseg_len = 0;
    e = sscan::launch_fwd_checkpoints_agg(p, bf16, s);
  } else {
    e = sscan::launch_fwd_checkpoints(p, bf16, s);
  }
  if (e != hipSuccess) return hip_fail(e, "checkpoint launch");
  }

  // 2. reverse pass and reductions
  sscan::BwdParams q{};
  q.x = x; q.dt = delta; q.z = z; q.B = B; q.C = C; q.dy = dy;
  q.A = A; q.Dskip = D; q.bias = delta_bias; q.dlast = dlast_state; q.ckpt = ckpt;
  q.dx = dx; q.ddt = ddelta; q.dz = dz;
  q.gB_part = reinterpret_cast<float*>(ws + lo.gB);
  q.gC_part = reinterpret_cast<float*>(ws + lo.gC);
  q.gA_part = reinterpret_cast<float*>(ws + lo.gA);
  q.gD_part = reinterpret_cast<float*>(ws + lo.gD);
  q.gbias_part = reinterpret_cast<float*>(ws + lo.gb);
  q.dh0 = dinitial_state;
  q.dB = dB; q.dC = dC; q.dA = dA; q.dD = dD; q.dbias = ddelta_bias;
  q.batch = batch; q.L = seqlen; q.dim = dim; q.ndtiles = ndt; q.nblk = nblk;
  q.N = static_cast<int>(N);
  q.euler = euler;
  q.nseg = lo.bseg;
  q.seg_blocks = lo.seg_blocks;
  q.ragg_g = reinterpret_cast<float*>(ws + lo.rg);
  q.ragg_s = reinterpret_cast<float*>(ws + lo.rs);
  q.gin = reinterpret_cast<float*>(ws + lo.gin);
  q.carry_done = agg_in_ckpt;
  q.agg_done = seg_agg;
  e = sscan::launch_bwd(q, bf16, s);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return ok();
}

int step_impl(int64_t batch, int64_t dim, int64_t dstate, int dtype, unsigned flags, float* state, const void* x,
              const void* delta, const float* A, const void* B, const void* C, const float* D, const void* z,
              const float* delta_bias, void* y, void* stream, int64_t dconv, const float* conv_w,
              const float* conv_b, float* conv_state) {
  int rc = check_common(batch, dim, dstate, dtype, flags);
  if (rc) return rc;
  rc = check_conv(ConvArgs{dconv, conv_w, conv_b, conv_state, conv_state}, batch, dim);
  if (rc) return rc;
  if (batch == 0 || dim == 0) return ok();
  if (conv_w && dconv > 1 && !conv_state)
    return fail(SSCAN_ERR_INVALID_ARG, "null required pointer (conv_state, dconv > 1)");
  if (!state || !x || !delta || !A || !B || !C || !y)
    return fail(SSCAN_ERR_INVALID_ARG, "null required pointer (state, x, delta, A, B, C and y are required)");
  const size_t es = dtype == SSCAN_BF16 ? 2 : 4;
  if (!aligned(x, es) || !aligned(delta, es) || !aligned(y, es) || (z && !aligned(z, es)) || !aligned(B, es) ||
      !aligned(C, es))
    return fail(SSCAN_ERR_INVALID_ARG, "token tensor not aligned to its element size");
  if (!aligned(state, 4) || !aligned(A, 4) || (D && !aligned(D, 4)) || (delta_bias && !aligned(delta_bias, 4)))
    return fail(SSCAN_ERR_INVALID_ARG, "float32 tensor not 4-byte aligned");
  const size_t tok = static_cast<size_t>(batch) * dim * es;
  const size_t st = static_cast<size_t>(batch) * dim * dstate * sizeof(float);
  const size_t bc = static_cast<size_t>(batch) * dstate * es;
  if (overlaps(y, tok, x, tok) || overlaps(y, tok, delta, tok) || overlaps(y, tok, z, tok) || overlaps(y, tok, state, st) ||
      overlaps(y, tok, B, bc) || overlaps(y, tok, C, bc))
    return fail(SSCAN_ERR_INVALID_ARG, "y overlaps an input or the state");
  if (overlaps(state, st, x, tok) || overlaps(state, st, delta, tok) || overlaps(state, st, z, tok) ||
      overlaps(state, st, B, bc) || overlaps(state, st, C, bc) || overlaps(state, st, A, dim * dstate * 4))
    return fail(SSCAN_ERR_INVALID_ARG, "state overlaps an input");
  sscan::StepParams p{};
  p.state = state; p.x = x; p.dt = delta; p.z = z; p.B = B; p.C = C;
  p.A = A; p.Dskip = D; p.bias = delta_bias; p.y = y;
  p.batch = batch; p.dim = dim; p.N = static_cast<int>(dstate);
  p.euler = (flags & SSCAN_FLAG_EULER) != 0;
  p.conv_w = conv_w; p.conv_b = conv_b; p.conv_state = conv_state; p.dconv = static_cast<int>(conv_w ? dconv : 1);
  if (conv_state) {
    const size_t cs = static_cast<size_t>(batch) * dim * (dconv - 1) * 4;
    if (overlaps(conv_state, cs, state, st) || overlaps(conv_state, cs, x, tok) || overlaps(conv_state, cs, y, tok))
      return fail(SSCAN_ERR_INVALID_ARG, "conv_state overlaps a tensor");
  }
  hipError_t e = sscan::launch_step(p, dtype == SSCAN_BF16, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "step launch");
  return ok();
}

}  // namespace

extern "C" {

int sscan_version(void) { return SSCAN_VERSION; }

const char* sscan_last_error(void) { return g_last_error.c_str(); }

size_t sscan_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype) {
  (void)dtype;
  if (batch <= 0 || seqlen <= 0 || dim <= 0 || dstate < 1 || dstate > SSCAN_MAX_DSTATE) return 0;
  const SegPlan pl = plan_segments(batch, seqlen, dim, dstate, 0, ~size_t(0), true);
  return seg_workspace_bytes(batch, dim, dstate, pl.nseg);
}

size_t sscan_fwd_segmented_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                                          int64_t num_segments) {
  (void)dtype;
  if (batch <= 0 || seqlen <= 0 || dim <= 0 || dstate < 1 || dstate > SSCAN_MAX_DSTATE || num_segments < 0) return 0;
  const SegPlan pl = plan_segments(batch, seqlen, dim, dstate, num_segments, ~size_t(0), true);
  return seg_workspace_bytes(batch, dim, dstate, pl.nseg);
}

sscan_status sscan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype, unsigned int flags,
                       const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
                       const void* z, const float* delta_bias, const float* initial_state, void* y, float* last_state,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return static_cast<sscan_status>(fwd_impl(batch, seqlen, dim, dstate, dtype, flags, x, delta, A, B, C, D, z, delta_bias, initial_state, y,
                  last_state, workspace, workspace_bytes, 0, stream, ConvArgs{}));
}

size_t sscan_checkpoint_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  if (batch <= 0 || seqlen <= 0 || dim <= 0 || dstate < 1 || dstate > SSCAN_MAX_DSTATE) return 0;
  return checkpoint_bytes(batch, seqlen, dim, dstate);
}

sscan_status sscan_fwd_checkpointed(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                                    unsigned int flags, const void* x, const void* delta, const float* A, const void* B,
                                    const void* C, const float* D, const void* z, const float* delta_bias,
                                    const float* initial_state, void* y, float* last_state, void* workspace,
                                    size_t workspace_bytes, float* checkpoints, size_t checkpoint_bytes_, void* stream) {
  if (!checkpoints && batch > 0 && seqlen > 0 && dim > 0)
    return static_cast<sscan_status>(fail(SSCAN_ERR_INVALID_ARG, "null required pointer (checkpoints)"));
  return static_cast<sscan_status>(fwd_impl(batch, seqlen, dim, dstate, dtype, flags, x, delta, A, B, C, D, z, delta_bias, initial_state, y,
                  last_state, workspace, workspace_bytes, 0, stream, ConvArgs{}, checkpoints, checkpoint_bytes_));
}

sscan_status sscan_fwd_conv(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int64_t dconv, int dtype,
                            unsigned int flags, const void* x, const float* conv_w, const float* conv_b,
                            const float* conv_state_in, float* conv_state_out, const void* delta, const float* A,
                            const void* B, const void* C, const float* D, const void* z, const float* delta_bias,
                            const float* initial_state, void* y, float* last_state, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!conv_w) return static_cast<sscan_status>(fail(SSCAN_ERR_INVALID_ARG, "null required pointer (conv_w)"));
  return static_cast<sscan_status>(fwd_impl(batch, seqlen, dim, dstate, dtype, flags, x, delta, A, B, C, D, z, delta_bias, initial_state, y,
                  last_state, workspace, workspace_bytes, 0, stream,
                  ConvArgs{dconv, conv_w, conv_b, conv_state_in, conv_state_out}));
}

sscan_status sscan_fwd_noalloc(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype, unsigned int flags,
                               const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
                               const void* z, const float* delta_bias, const float* initial_state, void* y,
                               float* last_state, void* stream) {
  // the split sscan_fwd would choose with an unlimited workspace; rejected if its
  // scratch exceeds the static array (nothing is launched then)
  const size_t need = sscan_fwd_workspace_size(batch, seqlen, dim, dstate, dtype);
  if (need > SSCAN_NOALLOC_SCRATCH_BYTES)
    return static_cast<sscan_status>(fail(SSCAN_ERR_INVALID_ARG,
                "sscan_fwd_noalloc: this shape needs %zu bytes of scratch, above the static %zu "
                "(SSCAN_NOALLOC_SCRATCH_BYTES); use sscan_fwd with a workspace",
                need, static_cast<size_t>(SSCAN_NOALLOC_SCRATCH_BYTES)));
  void* ws = nullptr;
  if (need > 0) {
    int rc = SSCAN_OK;
    ws = noalloc_scratch(&rc);
    if (!ws) return static_cast<sscan_status>(rc);
  }
  return static_cast<sscan_status>(fwd_impl(batch, seqlen, dim, dstate, dtype, flags, x, delta, A, B, C, D, z, delta_bias, initial_state, y,
                  last_state, ws, ws ? static_cast<size_t>(SSCAN_NOALLOC_SCRATCH_BYTES) : 0, 0, stream, ConvArgs{}));
}

sscan_status sscan_fwd_segmented(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                                 unsigned int flags, const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
                                 const void* z, const float* delta_bias, const float* initial_state, void* y,
                                 float* last_state, void* workspace, size_t workspace_bytes, int64_t num_segments,
                                 void* stream) {
  return static_cast<sscan_status>(fwd_impl(batch, seqlen, dim, dstate, dtype, flags, x, delta, A, B, C, D, z, delta_bias, initial_state, y,
                  last_state, workspace, workspace_bytes, num_segments, stream, ConvArgs{}));
}

sscan_status sscan_step(int64_t batch, int64_t dim, int64_t dstate, int dtype, unsigned int flags, float* state,
                        const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
                        const void* z, const float* delta_bias, void* y, void* stream) {
  return static_cast<sscan_status>(step_impl(batch, dim, dstate, dtype, flags, state, x, delta, A, B, C, D, z, delta_bias, y, stream, 0, nullptr,
                   nullptr, nullptr));
}

sscan_status sscan_step_conv(int64_t batch, int64_t dim, int64_t dstate, int64_t dconv, int dtype, unsigned int flags,
                             float* state, float* conv_state, const void* x, const float* conv_w, const float* conv_b,
                             const void* delta, const float* A, const void* B, const void* C, const float* D, const void* z,
                             const float* delta_bias, void* y, void* stream) {
  if (!conv_w) return static_cast<sscan_status>(fail(SSCAN_ERR_INVALID_ARG, "null required pointer (conv_w)"));
  return static_cast<sscan_status>(step_impl(batch, dim, dstate, dtype, flags, state, x, delta, A, B, C, D, z, delta_bias, y, stream, dconv,
                   conv_w, conv_b, conv_state));
}

size_t sscan_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype) {
  (void)dtype;
  if (batch <= 0 || seqlen <= 0 || dim <= 0 || dstate < 1 || dstate > SSCAN_MAX_DSTATE) return 0;
  return bwd_layout(batch, seqlen, dim, dstate).total;
}

sscan_status sscan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype, unsigned int flags,
                       const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
                       const void* z, const float* delta_bias, const float* initial_state, const void* dy,
                       const float* dlast_state, void* dx, void* ddelta, float* dA, void* dB, void* dC, float* dD,
                       void* dz, float* ddelta_bias, float* dinitial_state, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return static_cast<sscan_status>(bwd_impl(batch, seqlen, dim, dstate, dtype, flags, x, delta, A, B, C, D, z, delta_bias, initial_state, dy,
                  dlast_state, dx, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dinitial_state, workspace,
                  workspace_bytes, stream));
}

size_t sscan_bwd_checkpointed_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype) {
  (void)dtype;
  if (batch <= 0 || seqlen <= 0 || dim <= 0 || dstate < 1 || dstate > SSCAN_MAX_DSTATE) return 0;
  return bwd_layout(batch, seqlen, dim, dstate).total_saved;
}

sscan_status sscan_bwd_checkpointed(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype, unsigned int flags,
                                    const void* x, const void* delta, const float* A, const void* B, const void* C,
                                    const float* D, const void* z, const float* delta_bias, const float* checkpoints,
                                    size_t checkpoint_bytes_, const void* dy, const float* dlast_state, void* dx,
                                    void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz, float* ddelta_bias,
                                    float* dinitial_state, void* workspace, size_t workspace_bytes, void* stream) {
  return static_cast<sscan_status>(bwd_impl(batch, seqlen, dim, dstate, dtype, flags, x, delta, A, B, C, D, z, delta_bias, nullptr, dy,
                  dlast_state, dx, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dinitial_state, workspace,
                  workspace_bytes, stream, checkpoints, checkpoint_bytes_, true));
}

}  // extern "C"
