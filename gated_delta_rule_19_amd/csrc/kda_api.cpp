// Host side of the KDA C ABI: argument validation, the sequence-split planner,
// workspace layout, schedule upload and kernel launches.
//
// The planner follows "部署 Kimi K3：从 KDA Kernel 到 Fleet 调度", §1.2 (an
// intra-device context-parallel planner: cut a long sequence into segments,
// compute each segment's transition without knowing its entry state, then
// recover every entry state exactly) and §二 (the (M, S~) decomposition
// S = S~ + M S_in and its associative composition).  Work that would leave
// the device mostly idle -- a few heads of one long sequence -- is cut into
// chunk-aligned segments:
//   1. segment pass : for every segment but the last, its (M, S~) pair, by
//                     running the state-carrying kernel over [S~ | M] from
//                     [0 | I] with values [V | 0];
//   2. scan         : Sin[0] = S_0, Sin[j+1] = S~_j + M_j Sin[j];
//   3. replay       : every segment from its true entry state, writing o.
#include "kda.h"
#include "kda_internal.h"

#include <algorithm>
#include <climits>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

using namespace kda;

static_assert(kNoAllocScratchBytes == (size_t)KDA_NOALLOC_SCRATCH_BYTES,
              "the header's scratch size is the library's");
static_assert(sizeof(kda_prefill_options) == 64, "kda_prefill_options layout");

namespace {

// Automatic split policy: split only when the unsplit state-carrying work
// has fewer than kAutoMinChains workgroups (one per sequence-head), then aim
// for kAutoSegments segments of at least kAutoMinSegChunks chunks each.
constexpr int64_t kAutoMinChains = 64;
constexpr int64_t kAutoSegments = 64;
constexpr int64_t kAutoMinSegChunks = 4;
// Fewest (sequence, head) chains for the fused prefill kernel without a
// split (below that the fused planner or the two kernels fill the chip
// better), and fewest (segment, head) chains of an explicit planner split
// for its segment pass and replay to run on the fused kernel too.
constexpr int64_t kFusedMinChainHeads = 129;
constexpr int64_t kFusedSplitMinChainHeads = 256;

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned_elt(const void *p, kda_dtype dt) {
  return ((uintptr_t)p & (dt == KDA_BF16 ? 1u : 3u)) == 0;
}

// Whether the automatic cut is the fused planner's: bf16 calls with a
// chain count in [kFusedAutoMinChains, kFusedAutoMaxChains] on the automatic
// path.  It cuts a sequence into as many segments as keep each of the fused
// planner's two passes within one workgroup per compute unit (the first
// pass runs (segments - 1) x chains workgroups), at least
// kFusedMinSegChunks chunks each (shorter ones measured slower than the
// two kernels), and only when that gives 3 or more (two segments run one
// after the other, which the unsplit call already does).
constexpr int64_t kFusedAutoMinChains = 8, kFusedAutoMaxChains = 128;
constexpr int64_t kFusedMinSegChunks = 12;
bool fused_auto_cut(int32_t num_seqs, int32_t H, size_t es, int32_t path, int32_t split_hint) {
  const int64_t chains = (int64_t)num_seqs * H;
  return es == 2 && path == KDA_PATH_AUTO && split_hint == 0 &&
         chains >= kFusedAutoMinChains && chains <= kFusedAutoMaxChains;
}

int64_t plan_nseg(int64_t len, int32_t num_seqs, int32_t H, int32_t split_hint,
                  bool fused_cut = false) {
  if (len <= 0)
    return 1;
  const int64_t nch = (len + kC - 1) / kC;
  if (split_hint == 1)
    return 1;
  if (split_hint > 1)
    return std::min<int64_t>(split_hint, nch);
  const int64_t chains = (int64_t)num_seqs * H;
  if (fused_cut) {
    const int64_t n = std::min<int64_t>(1 + kComputeUnits / chains, nch / kFusedMinSegChunks);
    return n >= 3 ? n : 1;
  }
  if (chains >= kAutoMinChains)
    return 1;
  return std::max<int64_t>(1, std::min<int64_t>(kAutoSegments, nch / kAutoMinSegChunks));
}

ChainDesc chain(int64_t tok0, int64_t ntok, int64_t chunk0, int64_t init_idx,
                int64_t final_idx) {
  ChainDesc c;
  c.tok0 = tok0;
  c.ntok = (int32_t)ntok;
  c.chunk0 = (int32_t)chunk0;
  c.init_idx = (int32_t)init_idx;
  c.final_idx = (int32_t)final_idx;
  c.ckpt_chunk = c.ckpt_idx = -1;
  c.ckpt_last = -2;
  c.ckpt_every = 1;
  return c;
}

// The schedule for one call, built on the host.
struct Plan {
  std::vector<ChunkDesc> chunks;
  std::vector<ChainDesc> chains;    // prefill / replay (width dv, writes o)
  std::vector<ChainDesc> segchains; // segment pass (width dk + dv)
  std::vector<ChainDesc> headchains; // fused planner: first segments, run beside the segment pass
  std::vector<ScanDesc> scans;
  int64_t npairs = 0, nsin = 0;
  // bf16 without a planner split runs the fused kernel: no chunk-prep records
  bool fused = false;
  // bf16 with a planner split whose segment pass and replay run on the fused
  // kernel: no chunk-prep records either
  bool fused_split = false;
  // the fused path was asked for a call it cannot run (fp32)
  bool path_unsupported = false;
  // workspace layout
  size_t off_chunks = 0, off_chains = 0, off_seg = 0, off_head = 0, off_scan = 0,
         table_bytes = 0;
  size_t off_rec = 0, off_M = 0, off_St = 0, off_Sin = 0, total = 0;
};

void layout(Plan &p, int32_t H, size_t es) {
  size_t o = 0;
  p.off_chunks = o;
  o = align_up(o + p.chunks.size() * sizeof(ChunkDesc));
  p.off_chains = o;
  o = align_up(o + p.chains.size() * sizeof(ChainDesc));
  p.off_seg = o;
  o = align_up(o + p.segchains.size() * sizeof(ChainDesc));
  p.off_head = o;
  o = align_up(o + p.headchains.size() * sizeof(ChainDesc));
  p.off_scan = o;
  o = align_up(o + p.scans.size() * sizeof(ScanDesc));
  p.table_bytes = o;
  p.off_rec = o;
  if (!p.fused && !p.fused_split)
    o = align_up(o + p.chunks.size() * (size_t)H * k1_record_bytes(es));
  const size_t mat = (size_t)kD * kD * sizeof(float);
  p.off_M = o;
  o = align_up(o + (size_t)p.npairs * H * mat);
  p.off_St = o;
  o = align_up(o + (size_t)p.npairs * H * mat);
  p.off_Sin = o;
  o = align_up(o + (size_t)p.nsin * H * mat);
  p.total = o;
}

// Prefill schedule.  Returns false on bad cu_seqlens.
// Chunk count, from the sequence start, of sequence n's state checkpoint: the
// last position p with pos0 < p <= pos0 + len and p a multiple of align
// (pos0 and align multiples of the chunk length); 0 when there is none.
int64_t ckpt_chunks(int64_t pos0, int64_t len, int64_t align) {
  if (align <= 0)
    return 0;
  const int64_t p = (pos0 + len) / align * align;
  return p > pos0 ? (p - pos0) / kC : 0;
}

// Hash-aligned positions p with pos0 < p <= pos0 + len.
int64_t ckpt_count(int64_t pos0, int64_t len, int64_t align) {
  return align <= 0 ? 0 : (pos0 + len) / align - pos0 / align;
}

// The checkpoints of one sequence, as chunks counted from its first: chunk
// `first` (the one ending at the first checkpoint), then every `every`
// chunks, `count` of them.  all = false: only the last one.
struct SeqCkpts {
  int64_t first = -1, every = 1, count = 0;
};
SeqCkpts seq_ckpts(int64_t pos0, int64_t len, int64_t align, bool all) {
  SeqCkpts c;
  const int64_t n = ckpt_count(pos0, len, align);
  if (n <= 0)
    return c;
  if (!all) {
    c.first = ckpt_chunks(pos0, len, align) - 1;
    c.count = 1;
    return c;
  }
  c.first = ((pos0 / align + 1) * align - pos0) / kC - 1;
  c.every = align / kC;
  c.count = n;
  return c;
}

// Gives chain `c` (chunks [s0, s0 + cnt) of its sequence) the sequence's
// checkpoints that fall in it; idx0: the sequence's first checkpoint index.
void assign_ckpts(ChainDesc &c, const SeqCkpts &k, int64_t s0, int64_t cnt, int64_t idx0) {
  if (k.count <= 0)
    return;
  const int64_t last = k.first + (k.count - 1) * k.every;
  const int64_t j0 = s0 <= k.first ? 0 : (s0 - k.first + k.every - 1) / k.every;
  const int64_t c0 = k.first + j0 * k.every;
  const int64_t c1 = std::min(last, s0 + cnt - 1);
  if (c0 > c1)
    return;
  c.ckpt_chunk = (int32_t)(c0 - s0);
  c.ckpt_last = (int32_t)(c1 - s0);
  c.ckpt_every = (int32_t)k.every;
  c.ckpt_idx = (int32_t)(idx0 + j0);
}

// path: KDA_PATH_AUTO, KDA_PATH_TWO_KERNEL or KDA_PATH_FUSED
bool build_prefill_plan(int32_t N, const int64_t *cu, int32_t H, int32_t split_hint,
                        bool has_init, bool has_final, size_t es, Plan &p,
                        const int64_t *pos0 = nullptr, int64_t align = 0,
                        bool all_ckpts = false, int32_t path = KDA_PATH_AUTO,
                        bool layer_steps = false) {
  int64_t ckpt_base = 0; // first checkpoint index of the current sequence
  if (!cu || cu[0] != 0)
    return false;
  // asking for the fused kernel turns the automatic split off (an explicit
  // split runs the planner on it)
  if (path == KDA_PATH_FUSED && split_hint == 0)
    split_hint = 1;
  for (int32_t n = 0; n < N; ++n)
    if (cu[n + 1] < cu[n] || cu[n + 1] - cu[n] > INT32_MAX)
      return false;
  // The implementation.  bf16 with enough chains to give every compute unit
  // a few (sequence or segment, head) pairs: chunk prep and state carry run
  // fused in one kernel and no chunk-prep records go through memory.  With
  // fewer chains the chunk-parallel prep kernel keeps the whole chip busy
  // and the two-kernel path is faster.  A split on the fused kernel (the
  // fused planner) runs each split sequence's first segment from its known
  // entry state beside the segment pass of its middle segments, then the
  // scan, then the replay of all but the first segment.
  const bool fcut = fused_auto_cut(N, H, es, path, split_hint);
  std::vector<int64_t> nsegs(N);
  int64_t split_pairs = 0; // (segment, head) chains of the first pass / H
  for (int32_t n = 0; n < N; ++n) {
    nsegs[n] = plan_nseg(cu[n + 1] - cu[n], N, H, split_hint, fcut);
    split_pairs += nsegs[n] > 1 ? nsegs[n] - 1 : 0;
  }
  const bool split = split_pairs > 0;
  if (path == KDA_PATH_FUSED) {
    p.fused = es == 2 && !split;
    p.fused_split = es == 2 && split;
    p.path_unsupported = es != 2;
  } else if (path == KDA_PATH_AUTO) {
    p.fused = es == 2 && !split && (int64_t)N * H >= kFusedMinChainHeads;
    p.fused_split =
        es == 2 && split && (fcut || split_pairs * H >= kFusedSplitMinChainHeads);
  }
  for (int32_t n = 0; n < N; ++n) {
    const int64_t len = cu[n + 1] - cu[n];
    const int64_t nch = (len + kC - 1) / kC;
    const int64_t c0 = (int64_t)p.chunks.size();
    for (int64_t i = 0; i < nch; ++i) {
      ChunkDesc d;
      d.tok0 = cu[n] + i * kC;
      d.len = (int32_t)std::min<int64_t>(kC, cu[n + 1] - d.tok0);
      d.seq = n;
      p.chunks.push_back(d);
    }
    // the chunks after which checkpoint states are taken (last-only mode:
    // one per sequence, at index n; all: the sequence's run of indices)
    const SeqCkpts ck = seq_ckpts(pos0 ? pos0[n] : 0, len, align, all_ckpts);
    const int64_t idx0 = all_ckpts ? ckpt_base : n;
    ckpt_base += ck.count;
    const int64_t nseg = nsegs[n];
    if (nseg <= 1) {
      p.chains.push_back(chain(cu[n], len, c0, has_init ? n : -1, has_final ? n : -1));
      assign_ckpts(p.chains.back(), ck, 0, nch, idx0);
      continue;
    }
    // chunk-aligned segments of near-equal length.  On the fused planner the
    // first pass takes max(first, rho x the longest middle segment) chunk
    // steps and the replay the longest later segment, where rho is a
    // segment-pass step's cost over that of a step that carries the state
    // and o: about 0.9, and 0.83 with the layer steps on (the output norm
    // and gate run in the latter only).  The first segment's length
    // minimises the sum of the two passes (the shortest of the ties).  The
    // lengths do not change the workspace layout.
    int64_t first = -1;
    if (p.fused_split) {
      const double rho = layer_steps ? 0.83 : 0.9;
      double best = 0.0;
      for (int64_t f = 1; f + nseg - 1 <= nch; ++f) {
        const int64_t qm = (nch - f + nseg - 2) / (nseg - 1);
        const double c = std::max(static_cast<double>(f), rho * static_cast<double>(qm)) +
                         static_cast<double>(qm);
        if (first < 0 || c < best - 1e-9) {
          best = c;
          first = f;
        }
      }
    }
    const int64_t rest = p.fused_split ? nch - first : nch, nrest = p.fused_split ? nseg - 1 : nseg;
    const int64_t q = rest / nrest, r = rest % nrest;
    const int64_t pair0 = p.npairs, sin0 = p.nsin;
    for (int64_t j = 0; j < nseg; ++j) {
      // first chunk (relative to the sequence) and chunk count of segment j
      int64_t s0, cnt;
      if (p.fused_split) {
        const int64_t jj = j - 1;
        s0 = j == 0 ? 0 : first + jj * q + std::min(jj, r);
        cnt = j == 0 ? first : q + (jj < r ? 1 : 0);
      } else {
        s0 = j * q + std::min(j, r);
        cnt = q + (j < r ? 1 : 0);
      }
      const int64_t t0 = cu[n] + s0 * kC;
      const int64_t nt = std::min<int64_t>(cnt * kC, cu[n + 1] - t0);
      const bool last = j + 1 == nseg;
      if (p.fused_split) {
        // segment 0 from the known entry state, its exit state to Sin[sin0];
        // segments 1 .. nseg - 2 through the segment pass (pairs from pair0);
        // segments 1 .. nseg - 1 replayed from Sin[sin0 + j - 1]
        if (j == 0) {
          p.headchains.push_back(chain(t0, nt, c0 + s0, has_init ? n : -1, sin0));
          assign_ckpts(p.headchains.back(), ck, s0, cnt, idx0);
          continue;
        }
        if (!last)
          p.segchains.push_back(chain(t0, nt, c0 + s0, -1, pair0 + j - 1));
        p.chains.push_back(
            chain(t0, nt, c0 + s0, -2 - (sin0 + j - 1), (last && has_final) ? n : -1));
        assign_ckpts(p.chains.back(), ck, s0, cnt, idx0);
        continue;
      }
      if (!last)
        p.segchains.push_back(chain(t0, nt, c0 + s0, -1, pair0 + j));
      p.chains.push_back(chain(t0, nt, c0 + s0, -2 - (sin0 + j), (last && has_final) ? n : -1));
      assign_ckpts(p.chains.back(), ck, s0, cnt, idx0);
    }
    if (p.fused_split) {
      // entry states of segments 1 .. nseg - 1, from segment 1's in Sin[sin0]
      if (nseg > 2)
        p.scans.push_back(ScanDesc{(int32_t)pair0, (int32_t)(nseg - 1), (int32_t)sin0,
                                   kScanEntryInSin});
      p.npairs += nseg - 2;
      p.nsin += nseg - 1;
    } else {
      p.scans.push_back(ScanDesc{(int32_t)pair0, (int32_t)nseg, (int32_t)sin0,
                                 has_init ? n : -1});
      p.npairs += nseg - 1;
      p.nsin += nseg;
    }
  }
  // longest chains first, so the tail of the launch is short work
  auto longer = [](const ChainDesc &a, const ChainDesc &b) { return a.ntok > b.ntok; };
  std::stable_sort(p.chains.begin(), p.chains.end(), longer);
  std::stable_sort(p.segchains.begin(), p.segchains.end(), longer);
  std::stable_sort(p.headchains.begin(), p.headchains.end(), longer);
  layout(p, H, es);
  return true;
}

// Segment-transition schedule: every segment is one segment-pass chain whose
// exit pair goes to the caller's (S_tilde, M) at the segment's index.
bool build_segment_plan(int32_t S, const int64_t *cu, int32_t H, size_t es, Plan &p) {
  if (!cu || cu[0] != 0)
    return false;
  for (int32_t s = 0; s < S; ++s)
    if (cu[s + 1] < cu[s] || cu[s + 1] - cu[s] > INT32_MAX)
      return false;
  for (int32_t s = 0; s < S; ++s) {
    const int64_t len = cu[s + 1] - cu[s];
    const int64_t nch = (len + kC - 1) / kC;
    const int64_t c0 = (int64_t)p.chunks.size();
    for (int64_t i = 0; i < nch; ++i) {
      ChunkDesc d;
      d.tok0 = cu[s] + i * kC;
      d.len = (int32_t)std::min<int64_t>(kC, cu[s + 1] - d.tok0);
      d.seq = s;
      p.chunks.push_back(d);
    }
    p.segchains.push_back(chain(cu[s], len, c0, -1, s));
  }
  std::stable_sort(p.segchains.begin(), p.segchains.end(),
                   [](const ChainDesc &a, const ChainDesc &b) { return a.ntok > b.ntok; });
  layout(p, H, es);
  return true;
}

size_t elt_size(kda_dtype dt) { return dt == KDA_BF16 ? 2 : 4; }

// Limits that keep every index inside the kernels' int32 / grid ranges.
bool plan_fits(const Plan &p, int32_t H) {
  const int64_t lim = (int64_t)1 << 30;
  // the state chain's 1-D grid: (chains x heads, rounded up to 8) x up to 4
  // column blocks workgroups
  const int64_t pairs =
      (int64_t)std::max(p.chains.size(), p.segchains.size() + p.headchains.size()) * H;
  return (int64_t)p.chunks.size() < lim && (int64_t)p.chains.size() < lim &&
         (int64_t)p.segchains.size() < lim && (int64_t)p.scans.size() < lim &&
         H <= 65535 && p.npairs < lim && p.nsin < lim && (pairs + 8) * 4 < ((int64_t)1 << 31);
}

// ---- pinned staging for the schedule upload --------------------------------
// A pinned host buffer may only be reused once the copy that read it has
// finished; each buffer carries an event recorded right after its copy.
struct Staging {
  void *host = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  int device = -1;
  bool in_use = false;
};
std::mutex g_staging_mu;
std::vector<Staging *> g_staging;

Staging *staging_acquire(size_t bytes, int device) {
  std::lock_guard<std::mutex> lk(g_staging_mu);
  for (Staging *s : g_staging) {
    if (s->in_use || s->device != device || s->cap < bytes)
      continue;
    if (hipEventQuery(s->ev) != hipSuccess)
      continue;
    s->in_use = true;
    return s;
  }
  Staging *s = new Staging();
  s->device = device;
  s->cap = std::max<size_t>(bytes, 64 * 1024);
  if (hipHostMalloc(&s->host, s->cap, hipHostMallocDefault) != hipSuccess) {
    delete s;
    return nullptr;
  }
  if (hipEventCreateWithFlags(&s->ev, hipEventDisableTiming) != hipSuccess) {
    (void)hipHostFree(s->host);
    delete s;
    return nullptr;
  }
  s->in_use = true;
  g_staging.push_back(s);
  return s;
}

void staging_release(Staging *s) {
  std::lock_guard<std::mutex> lk(g_staging_mu);
  s->in_use = false;
}

// The schedule tables are copied from a pinned host buffer that later calls
// reuse, so a captured copy would read whatever a later call left there at
// each replay: calls that upload tables refuse a capturing stream (before
// anything is enqueued).
kda_status refuse_capture(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess)
    return KDA_ERR_HIP;
  return cs == hipStreamCaptureStatusNone ? KDA_OK : KDA_ERR_UNSUPPORTED;
}

// Copy the plan's tables into the workspace on `stream`.
hipError_t upload_tables(const Plan &p, void *ws, hipStream_t stream) {
  if (p.table_bytes == 0)
    return hipSuccess;
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess)
    return e;
  Staging *st = staging_acquire(p.table_bytes, device);
  if (!st)
    return hipErrorOutOfMemory;
  uint8_t *h = (uint8_t *)st->host;
  std::memset(h, 0, p.table_bytes);
  if (!p.chunks.empty())
    std::memcpy(h + p.off_chunks, p.chunks.data(), p.chunks.size() * sizeof(ChunkDesc));
  if (!p.chains.empty())
    std::memcpy(h + p.off_chains, p.chains.data(), p.chains.size() * sizeof(ChainDesc));
  if (!p.segchains.empty())
    std::memcpy(h + p.off_seg, p.segchains.data(), p.segchains.size() * sizeof(ChainDesc));
  if (!p.headchains.empty())
    std::memcpy(h + p.off_head, p.headchains.data(), p.headchains.size() * sizeof(ChainDesc));
  if (!p.scans.empty())
    std::memcpy(h + p.off_scan, p.scans.data(), p.scans.size() * sizeof(ScanDesc));
  e = hipMemcpyAsync(ws, h, p.table_bytes, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess)
    e = hipEventRecord(st->ev, stream);
  staging_release(st);
  return e;
}

} // namespace

namespace {

// The gated entry points' layer arguments, validated (KDA_OK or
// KDA_ERR_INVALID_ARG); `o` is the output the gate may not alias.
kda_status layer_steps(const float *A_log, float g_min, float qk_norm_eps, const void *out_gate,
                       const float *out_norm_weight, float out_norm_eps, const void *o,
                       Prologue &pro, Epilogue &epi) {
  if (A_log) {
    // the chunk kernels' bound: every 16-token cumulative log decay >= -80
    if (!(g_min >= -5.f && g_min < 0.f) || ((uintptr_t)A_log & 3u) != 0)
      return KDA_ERR_INVALID_ARG;
    pro.A_log = A_log;
    pro.g_min = g_min;
  }
  if (!(qk_norm_eps >= 0.f) || qk_norm_eps > 3.0e38f)
    return KDA_ERR_INVALID_ARG;
  pro.qk_eps = qk_norm_eps;
  if (out_gate) {
    if (!(out_norm_eps > 0.f) || out_norm_eps > 3.0e38f ||
        ((uintptr_t)out_norm_weight & 3u) != 0 || (o != nullptr && out_gate == o))
      return KDA_ERR_INVALID_ARG;
    epi.gate = out_gate;
    epi.weight = out_norm_weight;
    epi.eps = out_norm_eps;
  }
  return KDA_OK;
}

// kda_chunk_prefill, kda_chunk_prefill_ckpt (ckpt_align = 0: no checkpoints)
// and kda_chunk_prefill_gated (prologue / epilogue on)
kda_status prefill_impl(int32_t num_seqs, const int64_t *cu_seqlens_host, int32_t H, int32_t dk,
                        int32_t dv, kda_dtype dt, const void *q, const void *k, const void *v,
                        const void *g, const void *beta, const float *initial_state, void *o,
                        float *final_state, int32_t split_hint, const int64_t *pos0,
                        int32_t ckpt_align, float *ckpt, void *workspace,
                        size_t workspace_bytes, void *stream, const Prologue &pro = Prologue(),
                        const Epilogue &epi = Epilogue(), bool all_ckpts = false,
                        int32_t path = KDA_PATH_AUTO) {
  if (dk != kD || dv != kD || (dt != KDA_F32 && dt != KDA_BF16))
    return KDA_ERR_UNSUPPORTED;
  if (path != KDA_PATH_AUTO && path != KDA_PATH_TWO_KERNEL && path != KDA_PATH_FUSED)
    return KDA_ERR_INVALID_ARG;
  if (num_seqs < 0 || H < 1 || split_hint < 0 || !cu_seqlens_host)
    return KDA_ERR_INVALID_ARG;
  if (ckpt_align != 0) {
    if (ckpt_align < 0 || ckpt_align % kC != 0 || !ckpt || !aligned16(ckpt))
      return KDA_ERR_INVALID_ARG;
    for (int32_t n = 0; pos0 && n < num_seqs; ++n)
      if (pos0[n] < 0 || pos0[n] % kC != 0 || pos0[n] > ((int64_t)1 << 62))
        return KDA_ERR_INVALID_ARG;
  }
  Plan p;
  if (!build_prefill_plan(num_seqs, cu_seqlens_host, H, split_hint, initial_state != nullptr,
                          final_state != nullptr, elt_size(dt), p, pos0, ckpt_align,
                          all_ckpts, path, pro.on() || epi.on()))
    return KDA_ERR_INVALID_ARG;
  if (p.path_unsupported)
    return KDA_ERR_UNSUPPORTED;
  if (!plan_fits(p, H))
    return KDA_ERR_INVALID_ARG;
  const int64_t T = cu_seqlens_host[num_seqs];
  if (T > 0) {
    if (!q || !k || !v || !g || !beta || !o)
      return KDA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) ||
        !aligned_elt(beta, dt) || !aligned16(o))
      return KDA_ERR_INVALID_ARG;
  }
  if (!aligned16(initial_state) || !aligned16(final_state))
    return KDA_ERR_INVALID_ARG;
  if (T > 0 && epi.on() && !aligned_elt(epi.gate, dt))
    return KDA_ERR_INVALID_ARG;
  if (num_seqs == 0)
    return KDA_OK;
  if (p.total > 0) {
    if (!workspace || workspace_bytes < p.total || ((uintptr_t)workspace % kAlign) != 0)
      return KDA_ERR_WORKSPACE;
  }
  hipStream_t s = (hipStream_t)stream;
  if (const kda_status cs = refuse_capture(s); cs != KDA_OK)
    return cs;
  uint8_t *ws = (uint8_t *)workspace;
  const int elt = dt == KDA_BF16 ? 1 : 0;
  const ChunkDesc *d_chunks = (const ChunkDesc *)(ws + p.off_chunks);
  hipError_t e = upload_tables(p, ws, s);
  if (p.fused) {
    if (e == hipSuccess)
      e = launch_fused((const ChainDesc *)(ws + p.off_chains), (int32_t)p.chains.size(), H, q,
                        k, v, g, beta, o, initial_state, nullptr, final_state,
                        ckpt_align ? ckpt : nullptr, s, pro, epi);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
  }
  if (p.fused_split) {
    // first segments beside the segment pass, scan, replay: every pass that
    // carries a state on the fused kernel
    float *Sin = (float *)(ws + p.off_Sin);
    if (e == hipSuccess)
      e = launch_fused_pass1((const ChainDesc *)(ws + p.off_head), (int32_t)p.headchains.size(),
                             (const ChainDesc *)(ws + p.off_seg), (int32_t)p.segchains.size(),
                             H, q, k, v, g, beta, o, initial_state, Sin,
                             ckpt_align ? ckpt : nullptr, (float *)(ws + p.off_St),
                             (float *)(ws + p.off_M), s, pro, epi);
    if (e == hipSuccess)
      e = launch_scan(elt, (const ScanDesc *)(ws + p.off_scan), (int32_t)p.scans.size(), H,
                      (const float *)(ws + p.off_M), (const float *)(ws + p.off_St), nullptr,
                      Sin, s);
    if (e == hipSuccess)
      e = launch_fused((const ChainDesc *)(ws + p.off_chains), (int32_t)p.chains.size(), H, q,
                        k, v, g, beta, o, initial_state, (const float *)(ws + p.off_Sin),
                        final_state, ckpt_align ? ckpt : nullptr, s, pro, epi);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
  }
  if (e == hipSuccess)
    e = launch_k1(elt, d_chunks, (int32_t)p.chunks.size(), H, q, k, g, beta, ws + p.off_rec, pro,
                  s);
  if (e == hipSuccess && !p.segchains.empty()) {
    e = launch_k2(elt, 1, (const ChainDesc *)(ws + p.off_seg), (int32_t)p.segchains.size(), H,
                  ws + p.off_rec, v, nullptr, nullptr, nullptr, (float *)(ws + p.off_St),
                  (float *)(ws + p.off_M), /*m_scan_order=*/elt == 1 ? 2 : 1, Epilogue(), s);
    if (e == hipSuccess)
      e = launch_scan(elt, (const ScanDesc *)(ws + p.off_scan), (int32_t)p.scans.size(), H,
                      (const float *)(ws + p.off_M), (const float *)(ws + p.off_St),
                      initial_state, (float *)(ws + p.off_Sin), s);
  }
  // the output epilogue: in the replay pass's stores when it runs whole
  // rows, else as a pass of its own after it
  const bool epi_in_k2 = epi.on() && k2_fuses_epilogue((int32_t)p.chains.size(), H);
  if (e == hipSuccess)
    e = launch_k2(elt, 0, (const ChainDesc *)(ws + p.off_chains), (int32_t)p.chains.size(), H,
                  ws + p.off_rec, v, o, initial_state, (const float *)(ws + p.off_Sin),
                  final_state, ckpt_align ? ckpt : nullptr, 0, epi_in_k2 ? epi : Epilogue(),
                  s);
  if (e == hipSuccess && epi.on() && !epi_in_k2)
    e = launch_out_norm_gate(elt, T * H, o, epi, s);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

} // namespace

namespace {

kda_status decode_impl(int32_t N, int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                       const void *q, const void *k, const void *v, const void *g,
                       const void *beta, float *state, void *o, void *stream,
                       const Prologue &pro, const Epilogue &epi) {
  if (dk != kD || dv != kD || (dt != KDA_F32 && dt != KDA_BF16))
    return KDA_ERR_UNSUPPORTED;
  if (N < 0 || H < 1)
    return KDA_ERR_INVALID_ARG;
  if ((int64_t)N * H >= ((int64_t)1 << 31))
    return KDA_ERR_INVALID_ARG;
  if (N == 0)
    return KDA_OK;
  if (!q || !k || !v || !g || !beta || !state || !o)
    return KDA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) ||
      !aligned_elt(beta, dt) || !aligned16(state) || !aligned16(o))
    return KDA_ERR_INVALID_ARG;
  if (epi.on() && !aligned_elt(epi.gate, dt))
    return KDA_ERR_INVALID_ARG;
  const hipError_t e = launch_decode(dt == KDA_BF16 ? 1 : 0, N, H, q, k, v, g, beta, state, o,
                                     pro, epi, (hipStream_t)stream);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status replay_impl(int32_t N, int32_t H, int32_t dk, int32_t dv, kda_dtype dt, int32_t W,
                       const int32_t *accepted, const void *ck, const void *cv, const void *cg,
                       const void *cbeta, int32_t P, const void *q, const void *k,
                       const void *v, const void *g, const void *beta, float *state, void *o,
                       void *stream, const Prologue &pro, const Epilogue &epi) {
  if (dk != kD || dv != kD || (dt != KDA_F32 && dt != KDA_BF16))
    return KDA_ERR_UNSUPPORTED;
  if (N < 0 || H < 1 || W < 0 || W > KDA_REPLAY_MAX_TOKENS || P < 0 ||
      P > KDA_REPLAY_MAX_TOKENS)
    return KDA_ERR_INVALID_ARG;
  // token-row indices ((n W + t) H + h) kD stay within int64; blocks within 2^31
  if ((int64_t)N * H >= ((int64_t)1 << 31))
    return KDA_ERR_INVALID_ARG;
  if (N == 0)
    return KDA_OK;
  if (!accepted || !state || !aligned16(state) || ((uintptr_t)accepted & 3))
    return KDA_ERR_INVALID_ARG;
  if (W > 0 && (!ck || !cv || !cg || !cbeta || !aligned16(ck) || !aligned16(cv) ||
                !aligned16(cg) || !aligned_elt(cbeta, dt)))
    return KDA_ERR_INVALID_ARG;
  if (P > 0 && (!q || !k || !v || !g || !beta || !o || !aligned16(q) || !aligned16(k) ||
                !aligned16(v) || !aligned16(g) || !aligned_elt(beta, dt) || !aligned16(o)))
    return KDA_ERR_INVALID_ARG;
  if (P > 0 && epi.on() && !aligned_elt(epi.gate, dt))
    return KDA_ERR_INVALID_ARG;
  const hipError_t e = launch_replay(dt == KDA_BF16 ? 1 : 0, N, H, W, accepted, ck, cv, cg,
                                     cbeta, P, q, k, v, g, beta, state, o, pro, epi,
                                     (hipStream_t)stream);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

} // namespace

extern "C" {

const char *kda_status_string(kda_status s) {
  switch (s) {
  case KDA_OK:
    return "KDA_OK";
  case KDA_ERR_INVALID_ARG:
    return "KDA_ERR_INVALID_ARG";
  case KDA_ERR_UNSUPPORTED:
    return "KDA_ERR_UNSUPPORTED";
  case KDA_ERR_WORKSPACE:
    return "KDA_ERR_WORKSPACE";
  case KDA_ERR_HIP:
    return "KDA_ERR_HIP";
  default:
    return "KDA_ERR_UNKNOWN";
  }
}

int32_t kda_version(void) { return 100; }

int32_t kda_plan_num_segments(int64_t seq_len, int32_t num_seqs, int32_t H, int32_t split_hint) {
  return kda_plan_num_segments_dt(seq_len, num_seqs, H, split_hint, KDA_F32);
}

int32_t kda_plan_num_segments_dt(int64_t seq_len, int32_t num_seqs, int32_t H,
                                 int32_t split_hint, kda_dtype dt) {
  if (num_seqs < 0 || H < 1 || split_hint < 0 || (dt != KDA_F32 && dt != KDA_BF16))
    return KDA_ERR_INVALID_ARG;
  const int64_t n = plan_nseg(seq_len, num_seqs, H, split_hint,
                              fused_auto_cut(num_seqs, H, elt_size(dt), KDA_PATH_AUTO,
                                             split_hint));
  return (int32_t)std::min<int64_t>(n, INT32_MAX);
}

size_t kda_chunk_prefill_ex_workspace_size(int32_t num_seqs, const int64_t *cu_seqlens_host,
                                           int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                                           int32_t split_hint, const kda_prefill_options *opts) {
  const int32_t path = opts ? opts->path : KDA_PATH_AUTO;
  if (num_seqs < 0 || H < 1 || dk != kD || dv != kD || (dt != KDA_F32 && dt != KDA_BF16) ||
      split_hint < 0 || (path != KDA_PATH_AUTO && path != KDA_PATH_TWO_KERNEL &&
                         path != KDA_PATH_FUSED))
    return 0;
  Plan p;
  // has_init / has_final and the checkpoint and layer options do not change
  // the layout
  if (!build_prefill_plan(num_seqs, cu_seqlens_host, H, split_hint, false, true, elt_size(dt),
                          p, nullptr, 0, false, path) ||
      p.path_unsupported)
    return 0;
  return p.total;
}

size_t kda_chunk_prefill_workspace_size(int32_t num_seqs, const int64_t *cu_seqlens_host,
                                        int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                                        int32_t split_hint) {
  return kda_chunk_prefill_ex_workspace_size(num_seqs, cu_seqlens_host, H, dk, dv, dt,
                                             split_hint, nullptr);
}

kda_status kda_chunk_prefill_ex(int32_t num_seqs, const int64_t *cu_seqlens_host, int32_t H,
                                int32_t dk, int32_t dv, kda_dtype dt, const void *q,
                                const void *k, const void *v, const void *g, const void *beta,
                                const float *initial_state, void *o, float *final_state,
                                int32_t split_hint, const kda_prefill_options *opts,
                                void *workspace, size_t workspace_bytes, void *stream) {
  kda_prefill_options d;
  std::memset(&d, 0, sizeof(d));
  d.g_min = -5.f;
  d.out_norm_eps = 1e-6f;
  const kda_prefill_options &op = opts ? *opts : d;
  Prologue pro;
  Epilogue epi;
  const kda_status st = layer_steps(op.A_log, op.g_min, op.qk_norm_eps, op.out_gate,
                                    op.out_norm_weight, op.out_norm_eps, o, pro, epi);
  if (st != KDA_OK)
    return st;
  if (op.ckpt_align < 0 || (op.ckpt_all != 0 && op.ckpt_all != 1))
    return KDA_ERR_INVALID_ARG;
  float *ckpt = op.ckpt_align > 0 ? op.ckpt_state : nullptr;
  int32_t align = op.ckpt_align;
  if (align > 0 && op.ckpt_all) {
    const int64_t n = kda_prefill_num_checkpoints(num_seqs, cu_seqlens_host, op.pos0_host,
                                                  align);
    if (n < 0 || n > INT32_MAX / 2)
      return KDA_ERR_INVALID_ARG;
    if (n == 0) { // nothing to write: the states need no buffer
      align = 0;
      ckpt = nullptr;
    }
  }
  return prefill_impl(num_seqs, cu_seqlens_host, H, dk, dv, dt, q, k, v, g, beta, initial_state,
                      o, final_state, split_hint, align ? op.pos0_host : nullptr, align, ckpt,
                      workspace, workspace_bytes, stream, pro, epi, op.ckpt_all != 0, op.path);
}


kda_status kda_chunk_prefill(int32_t num_seqs, const int64_t *cu_seqlens_host, int32_t H,
                             int32_t dk, int32_t dv, kda_dtype dt, const void *q, const void *k,
                             const void *v, const void *g, const void *beta,
                             const float *initial_state, void *o, float *final_state,
                             int32_t split_hint, void *workspace, size_t workspace_bytes,
                             void *stream) {
  return prefill_impl(num_seqs, cu_seqlens_host, H, dk, dv, dt, q, k, v, g, beta, initial_state,
                      o, final_state, split_hint, nullptr, 0, nullptr, workspace,
                      workspace_bytes, stream);
}

kda_status kda_chunk_prefill_ckpt(int32_t num_seqs, const int64_t *cu_seqlens_host, int32_t H,
                                  int32_t dk, int32_t dv, kda_dtype dt, const void *q,
                                  const void *k, const void *v, const void *g, const void *beta,
                                  const float *initial_state, void *o, float *final_state,
                                  int32_t split_hint, const int64_t *pos0_host,
                                  int32_t ckpt_align, float *ckpt_state, void *workspace,
                                  size_t workspace_bytes, void *stream) {
  if (ckpt_align <= 0)
    return KDA_ERR_INVALID_ARG;
  return prefill_impl(num_seqs, cu_seqlens_host, H, dk, dv, dt, q, k, v, g, beta, initial_state,
                      o, final_state, split_hint, pos0_host, ckpt_align, ckpt_state, workspace,
                      workspace_bytes, stream);
}

kda_status kda_chunk_prefill_noalloc(int32_t num_seqs, const int64_t *cu_seqlens_host, int32_t H,
                                     int32_t dk, int32_t dv, kda_dtype dt, const void *q,
                                     const void *k, const void *v, const void *g,
                                     const void *beta, const float *initial_state, void *o,
                                     float *final_state, void *stream) {
  if (dk != kD || dv != kD || dt != KDA_BF16)
    return KDA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || H < 1 || !cu_seqlens_host)
    return KDA_ERR_INVALID_ARG;
  Plan p;
  if (!build_prefill_plan(num_seqs, cu_seqlens_host, H, 0, initial_state != nullptr,
                          final_state != nullptr, 2, p, nullptr, 0, false, KDA_PATH_FUSED))
    return KDA_ERR_INVALID_ARG;
  if (p.path_unsupported || !p.fused || !plan_fits(p, H))
    return KDA_ERR_INVALID_ARG;
  const int64_t T = cu_seqlens_host[num_seqs];
  if (T > 0) {
    if (!q || !k || !v || !g || !beta || !o)
      return KDA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) ||
        !aligned_elt(beta, dt) || !aligned16(o))
      return KDA_ERR_INVALID_ARG;
  }
  if (!aligned16(initial_state) || !aligned16(final_state))
    return KDA_ERR_INVALID_ARG;
  // the schedule must fit the fixed scratch (no workspace argument)
  if (p.total > kNoAllocScratchBytes)
    return KDA_ERR_WORKSPACE;
  if (num_seqs == 0)
    return KDA_OK;
  void *scr = nullptr;
  hipError_t e = noalloc_scratch(&scr);
  if (e != hipSuccess)
    return KDA_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  {
    // The tables go up from a fixed host buffer.  A copy from pageable host
    // memory has read its source when hipMemcpyAsync returns, so the buffer
    // is free again for the next call (the lock orders host threads).
    static std::mutex mu;
    static uint8_t host[kNoAllocScratchBytes];
    std::lock_guard<std::mutex> lk(mu);
    std::memset(host, 0, p.table_bytes);
    if (!p.chains.empty())
      std::memcpy(host + p.off_chains, p.chains.data(), p.chains.size() * sizeof(ChainDesc));
    e = hipMemcpyAsync(scr, host, p.table_bytes, hipMemcpyHostToDevice, s);
  }
  if (e == hipSuccess)
    e = launch_fused((const ChainDesc *)((uint8_t *)scr + p.off_chains),
                      (int32_t)p.chains.size(), H, q, k, v, g, beta, o, initial_state,
                      nullptr, final_state, nullptr, s);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int64_t kda_prefill_num_checkpoints(int32_t num_seqs, const int64_t *cu_seqlens_host,
                                    const int64_t *pos0_host, int32_t ckpt_align) {
  if (num_seqs < 0 || !cu_seqlens_host || cu_seqlens_host[0] != 0 || ckpt_align <= 0 ||
      ckpt_align % kC != 0)
    return -1;
  int64_t total = 0;
  for (int32_t n = 0; n < num_seqs; ++n) {
    const int64_t len = cu_seqlens_host[n + 1] - cu_seqlens_host[n];
    const int64_t p0 = pos0_host ? pos0_host[n] : 0;
    if (len < 0 || p0 < 0 || p0 % kC != 0 || p0 > ((int64_t)1 << 62))
      return -1;
    total += ckpt_count(p0, len, ckpt_align);
  }
  return total;
}

kda_status kda_chunk_prefill_ckpt_all(int32_t num_seqs, const int64_t *cu_seqlens_host,
                                      int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                                      const void *q, const void *k, const void *v,
                                      const void *g, const void *beta,
                                      const float *initial_state, void *o, float *final_state,
                                      int32_t split_hint, const int64_t *pos0_host,
                                      int32_t ckpt_align, float *ckpt_states, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  if (ckpt_align <= 0)
    return KDA_ERR_INVALID_ARG;
  const int64_t n = kda_prefill_num_checkpoints(num_seqs, cu_seqlens_host, pos0_host,
                                                ckpt_align);
  if (n < 0 || n > INT32_MAX / 2)
    return KDA_ERR_INVALID_ARG;
  if (n == 0) // nothing to write: the states need no buffer
    return prefill_impl(num_seqs, cu_seqlens_host, H, dk, dv, dt, q, k, v, g, beta,
                        initial_state, o, final_state, split_hint, nullptr, 0, nullptr,
                        workspace, workspace_bytes, stream);
  return prefill_impl(num_seqs, cu_seqlens_host, H, dk, dv, dt, q, k, v, g, beta, initial_state,
                      o, final_state, split_hint, pos0_host, ckpt_align, ckpt_states, workspace,
                      workspace_bytes, stream, Prologue(), Epilogue(), /*all_ckpts=*/true);
}

kda_status kda_chunk_prefill_gated(int32_t num_seqs, const int64_t *cu_seqlens_host, int32_t H,
                                   int32_t dk, int32_t dv, kda_dtype dt, const void *q,
                                   const void *k, const void *v, const void *g, const void *beta,
                                   const float *A_log, float g_min, float qk_norm_eps,
                                   const void *out_gate, const float *out_norm_weight,
                                   float out_norm_eps, const float *initial_state, void *o,
                                   float *final_state, int32_t split_hint, void *workspace,
                                   size_t workspace_bytes, void *stream) {
  Prologue pro;
  Epilogue epi;
  const kda_status st = layer_steps(A_log, g_min, qk_norm_eps, out_gate, out_norm_weight,
                                    out_norm_eps, o, pro, epi);
  if (st != KDA_OK)
    return st;
  return prefill_impl(num_seqs, cu_seqlens_host, H, dk, dv, dt, q, k, v, g, beta, initial_state,
                      o, final_state, split_hint, nullptr, 0, nullptr, workspace,
                      workspace_bytes, stream, pro, epi);
}

kda_status kda_decode_step(int32_t N, int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                           const void *q, const void *k, const void *v, const void *g,
                           const void *beta, float *state, void *o, void *stream) {
  return decode_impl(N, H, dk, dv, dt, q, k, v, g, beta, state, o, stream, Prologue(),
                     Epilogue());
}

kda_status kda_decode_step_gated(int32_t N, int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                                 const void *q, const void *k, const void *v, const void *g,
                                 const void *beta, const float *A_log, float g_min,
                                 float qk_norm_eps, const void *out_gate,
                                 const float *out_norm_weight, float out_norm_eps,
                                 float *state, void *o, void *stream) {
  Prologue pro;
  Epilogue epi;
  const kda_status st = layer_steps(A_log, g_min, qk_norm_eps, out_gate, out_norm_weight,
                                    out_norm_eps, o, pro, epi);
  if (st != KDA_OK)
    return st;
  return decode_impl(N, H, dk, dv, dt, q, k, v, g, beta, state, o, stream, pro, epi);
}

kda_status kda_decode_replay(int32_t N, int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                             int32_t W, const int32_t *accepted, const void *ck, const void *cv,
                             const void *cg, const void *cbeta, int32_t P, const void *q,
                             const void *k, const void *v, const void *g, const void *beta,
                             float *state, void *o, void *stream) {
  return replay_impl(N, H, dk, dv, dt, W, accepted, ck, cv, cg, cbeta, P, q, k, v, g, beta,
                     state, o, stream, Prologue(), Epilogue());
}

kda_status kda_decode_replay_gated(int32_t N, int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                                   int32_t W, const int32_t *accepted, const void *ck,
                                   const void *cv, const void *cg, const void *cbeta, int32_t P,
                                   const void *q, const void *k, const void *v, const void *g,
                                   const void *beta, const float *A_log, float g_min,
                                   float qk_norm_eps, const void *out_gate,
                                   const float *out_norm_weight, float out_norm_eps,
                                   float *state, void *o, void *stream) {
  Prologue pro;
  Epilogue epi;
  const kda_status st = layer_steps(A_log, g_min, qk_norm_eps, out_gate, out_norm_weight,
                                    out_norm_eps, o, pro, epi);
  if (st != KDA_OK)
    return st;
  return replay_impl(N, H, dk, dv, dt, W, accepted, ck, cv, cg, cbeta, P, q, k, v, g, beta,
                     state, o, stream, pro, epi);
}

size_t kda_segment_transition_workspace_size(int32_t num_segs,
                                             const int64_t *cu_seglens_host, int32_t H,
                                             int32_t dk, int32_t dv, kda_dtype dt) {
  if (num_segs < 0 || H < 1 || dk != kD || dv != kD || (dt != KDA_F32 && dt != KDA_BF16))
    return 0;
  Plan p;
  if (!build_segment_plan(num_segs, cu_seglens_host, H, elt_size(dt), p))
    return 0;
  return p.total;
}

kda_status kda_segment_transition(int32_t num_segs, const int64_t *cu_seglens_host, int32_t H,
                                  int32_t dk, int32_t dv, kda_dtype dt, const void *k,
                                  const void *v, const void *g, const void *beta, float *M,
                                  float *S_tilde, void *workspace, size_t workspace_bytes,
                                  void *stream) {
  if (dk != kD || dv != kD || (dt != KDA_F32 && dt != KDA_BF16))
    return KDA_ERR_UNSUPPORTED;
  if (num_segs < 0 || H < 1 || !cu_seglens_host)
    return KDA_ERR_INVALID_ARG;
  Plan p;
  if (!build_segment_plan(num_segs, cu_seglens_host, H, elt_size(dt), p))
    return KDA_ERR_INVALID_ARG;
  if (!plan_fits(p, H))
    return KDA_ERR_INVALID_ARG;
  const int64_t T = cu_seglens_host[num_segs];
  if (T > 0) {
    if (!k || !v || !g || !beta)
      return KDA_ERR_INVALID_ARG;
    if (!aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned_elt(beta, dt))
      return KDA_ERR_INVALID_ARG;
  }
  if (num_segs > 0 && (!M || !S_tilde))
    return KDA_ERR_INVALID_ARG;
  if (!aligned16(M) || !aligned16(S_tilde))
    return KDA_ERR_INVALID_ARG;
  if (num_segs > 0) {
    const size_t bytes = (size_t)num_segs * H * kD * kD * sizeof(float);
    const uint8_t *a = (const uint8_t *)M, *b = (const uint8_t *)S_tilde;
    if (a < b + bytes && b < a + bytes)
      return KDA_ERR_INVALID_ARG;
  }
  if (num_segs == 0)
    return KDA_OK;
  if (p.total > 0) {
    if (!workspace || workspace_bytes < p.total || ((uintptr_t)workspace % kAlign) != 0)
      return KDA_ERR_WORKSPACE;
  }
  hipStream_t s = (hipStream_t)stream;
  if (const kda_status cs = refuse_capture(s); cs != KDA_OK)
    return cs;
  uint8_t *ws = (uint8_t *)workspace;
  const int elt = dt == KDA_BF16 ? 1 : 0;
  const ChunkDesc *d_chunks = (const ChunkDesc *)(ws + p.off_chunks);
  hipError_t e = upload_tables(p, ws, s);
  if (e == hipSuccess)
    e = launch_k1(elt, d_chunks, (int32_t)p.chunks.size(), H, nullptr, k, g, beta,
                  ws + p.off_rec, Prologue(), s);
  if (e == hipSuccess)
    e = launch_k2(elt, 1, (const ChainDesc *)(ws + p.off_seg), (int32_t)p.segchains.size(), H,
                  ws + p.off_rec, v, nullptr, nullptr, nullptr, S_tilde, M, 0, Epilogue(), s);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_segment_scan(int32_t num_segs, int32_t H, int32_t dk, int32_t dv, const float *M,
                            const float *S_tilde, const float *initial_state, float *S_in,
                            void *stream) {
  if (dk != kD || dv != kD)
    return KDA_ERR_UNSUPPORTED;
  // (the scan's descriptor counts num_segs + 1 states in an int32)
  if (num_segs < 0 || num_segs > INT32_MAX - 1 || H < 1 || H > (1 << 24) || !S_in ||
      !aligned16(S_in) || !aligned16(initial_state))
    return KDA_ERR_INVALID_ARG;
  if (num_segs > 0 && (!M || !S_tilde || !aligned16(M) || !aligned16(S_tilde)))
    return KDA_ERR_INVALID_ARG;
  const int64_t mat = (int64_t)H * kD * kD * (int64_t)sizeof(float);
  if ((int64_t)num_segs + 1 > INT64_MAX / 2 / mat)
    return KDA_ERR_INVALID_ARG;
  // S_in is written while the pairs and the initial state are read
  const uint8_t *out = (const uint8_t *)S_in;
  const int64_t out_bytes = ((int64_t)num_segs + 1) * mat;
  auto overlaps = [&](const float *in, int64_t bytes) {
    const uint8_t *a = (const uint8_t *)in;
    return in && bytes > 0 && a < out + out_bytes && out < a + bytes;
  };
  if (overlaps(M, num_segs * mat) || overlaps(S_tilde, num_segs * mat) ||
      overlaps(initial_state, mat))
    return KDA_ERR_INVALID_ARG;
  const hipError_t e = launch_scan_rows(num_segs, H, M, S_tilde, initial_state, S_in,
                                        (hipStream_t)stream);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

} // extern "C"
