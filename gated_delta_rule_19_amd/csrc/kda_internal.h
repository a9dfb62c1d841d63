// Host/device shared schedule records and kernel launchers (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

constexpr int kC = 64;  // chunk length
constexpr int kD = 128; // dk = dv

// One C-token chunk of one sequence (or segment).
struct ChunkDesc {
  int64_t tok0;  // first token (packed index)
  int32_t len;   // 1..64 valid tokens
  int32_t seq;   // owning sequence
};
static_assert(sizeof(ChunkDesc) == 16, "ChunkDesc layout");

// One state-carrying chain: a run of consecutive chunks of one sequence,
// tokens [tok0, tok0 + ntok), processed in order from an entry state to an
// exit state.  Its chunks' prep records are chunk0, chunk0 + 1, ...
//   init_idx >= 0  : entry state = user initial_state[init_idx]
//   init_idx == -1 : entry state = 0 (segment pass: [0 | I])
//   init_idx <= -2 : entry state = planner entry state Sin[-2 - init_idx]
//   final_idx >= 0 : exit state written at index final_idx of the output base
//   checkpoints    : the states after the chain's chunks ckpt_chunk,
//                    ckpt_chunk + ckpt_every, ... up to ckpt_last (counted
//                    from the chain's first chunk) are also written, at
//                    indices ckpt_idx, ckpt_idx + 1, ... of the checkpoint
//                    output; none when ckpt_last < ckpt_chunk
struct ChainDesc {
  int64_t tok0;
  int32_t ntok;
  int32_t chunk0;
  int32_t init_idx;
  int32_t final_idx;
  int32_t ckpt_chunk, ckpt_last, ckpt_every, ckpt_idx;
};
static_assert(sizeof(ChainDesc) == 40, "ChainDesc layout");

// One split sequence for the planner's prefix scan.
struct ScanDesc {
  int32_t pair0;    // index of segment 0's (M, S~) pair
  int32_t nseg;     // segments of this sequence (>= 2)
  int32_t sin0;     // index of segment 0's entry state in Sin
  int32_t init_idx; // user initial_state index, -1 for zero, or kScanEntryInSin
};
// ScanDesc::init_idx of a scan whose first entry state is already in
// Sin[sin0] (bf16 scan only)
constexpr int32_t kScanEntryInSin = -3;
static_assert(sizeof(ScanDesc) == 16, "ScanDesc layout");

// Column order of the chunk-prep record's MFMA A operands.  Inside each group
// of 32 logical columns k the element sits at physical position
//   p(k) = 8 * ((k % 16) / 4) + 4 * (k / 16) + k % 4,
// so the 8 consecutive elements at 8g .. 8g+7 hold logical columns
// 4g .. 4g+3 and 16+4g .. 16+4g+3.  Those are exactly the rows that lane
// group g holds in two stacked 16-row MFMA accumulator tiles, so an
// accumulator can be fed back as the B operand of the next product without
// moving data between lanes.
__host__ __device__ constexpr int kperm(int k) {
  return (k & ~31) | (((k & 15) >> 2) << 3) | ((k & 16) >> 2) | (k & 3);
}

// Inverse of kperm: the logical column held at physical position p.
__host__ __device__ constexpr int kperm_inv(int p) {
  return (p & ~31) | ((p & 4) << 2) | ((p & 24) >> 1) | (p & 3);
}

// Bytes of the chunk-prep record for one (chunk, head), element size es:
//   Q_decay [C][D], K_decay [C][D], K_restore^T [D][C], INV*Diag(beta) [C][C],
//   M_qk [C][C] (all of the element type, token columns in kperm order),
//   a_last [D] fp32; 256-aligned.  fp32 records keep Q_decay / K_decay
//   columns in kperm order and the state rows in channel order; bf16 records
//   the reverse, and store Q_decay, K_decay and M_qk in 16-byte pieces in
//   the order the bf16 prep writes them (kda_prep.hip).  bf16 records hold
//   the two lower-triangular C x C matrices as their nonzero 1 KiB fragment
//   blocks only (tri_block).
constexpr int kTriBlocks = 6; // nonzero (16-row, 32-token) blocks of a lower-triangular C x C
constexpr size_t k1_record_bytes(size_t es) {
  return es == 2 ? ((3 * 64 * 128 + 2 * kTriBlocks * 512) * es + 128 * 4 + 255) / 256 * 256
                 : ((3 * 64 * 128 + 2 * 64 * 64) * es + 128 * 4 + 255) / 256 * 256;
}

// A lower-triangular C x C matrix (INV Diag(beta), M_qk) in a bf16 record:
// its 16-row by 32-token fragment blocks b = 2 (row tile) + (token half),
// of which blocks 1 and 3 (row tiles 0 and 1 against tokens 32..63) lie
// wholly above the diagonal and are not stored.  The stored block index of
// block b, or -1 for those two.
__host__ __device__ constexpr int tri_block(int b) {
  return b == 0 ? 0 : (b == 2 ? 1 : (b >= 4 ? b - 2 : -1));
}

// Column blocks of the state-carrying kernel (columns of S per workgroup;
// each of its waves carries NCT 16-column tiles).  The wide block reads each
// chunk record once per head; the narrow one doubles the workgroups (each
// record is then read twice) for launches with too few chains to give every
// compute unit one workgroup.  The planner's segment pass over many segments
// is throughput-bound: there, 64-column blocks with one record buffer let two
// workgroups share a compute unit, each hiding the other's record loads.
constexpr int kBVWide = 128;
constexpr int kBVNarrow = 64;
constexpr int kK2ThroughputGroups = 512; // wide workgroups from which the segment pass uses it
constexpr int kK2ThroughputBV = 64;
constexpr int kK2ThroughputNCT = 1;
constexpr int k2_threads(int bv, int nct) { return bv / (16 * nct) * 64; }
constexpr int kComputeUnits = 256;
// Column block of the planner scan kernels.
constexpr int kScanBV = 16;

// Position of M[r][m] (r: output row, m: reduction index) in the scan order
// the planner's segment pass writes its transition matrices in for fp32
// calls: 1 KiB blocks, one per (wave w = r / 32, k-group i = m / 16, row
// tile t = r / 16 % 2) in that order, each holding the 64 lanes' A operands
// of the fp32 scan kernel's
// v_mfma_f32_16x16x4f32 products (lane 16 (m / 4 % 4) + r % 16, four
// consecutive reduction indices per lane).  One scan load is then 1 KiB
// contiguous.
__host__ __device__ constexpr int scan_m_index(int r, int m) {
  return ((((r >> 5) * 8 + (m >> 4)) * 2 + ((r >> 4) & 1)) * 64 + ((m >> 2) & 3) * 16 +
          (r & 15)) * 4 + (m & 3);
}

// bf16 planners hold M_j as two bf16 matrices, hi = bf16(M) and lo =
// bf16(M - hi), hi at elements [0, dk^2) and lo at [dk^2, 2 dk^2) of the
// same 64 KiB slot, each in the order of the bf16 scan kernel's
// v_mfma_f32_16x16x32_bf16 A operands: 1 KiB blocks per (wave w = r / 32,
// k-step s = m / 32, row tile t = r / 16 % 2) in that order, lane
// 16 (m / 8 % 4) + r % 16 holding the eight reduction indices
// m / 8 * 8 .. + 7.
__host__ __device__ constexpr int scan_m_bf16_index(int r, int m) {
  return ((((r >> 5) * 4 + (m >> 5)) * 2 + ((r >> 4) & 1)) * 64 + ((m >> 3) & 3) * 16 +
          (r & 15)) * 8 + (m & 7);
}

// Steps of the layer fused into the chunk prep ("Kimi K3.1 Pro 架构完全拆解"
// §3.2; "Kimi K3 的架構" §七):
//   A_log != null : the g input holds raw gate logits z, and the log decay is
//                   g_min * sigmoid(exp(A_log[h]) * z) (rows past a chunk's
//                   end decay by nothing);
//   qk_eps > 0    : q and k rows are L2-normalized, x / sqrt(sum x^2 + qk_eps).
struct Prologue {
  const float *A_log = nullptr;
  float g_min = -5.f;
  float qk_eps = 0.f;
  bool on() const { return A_log != nullptr || qk_eps > 0.f; }
};

// Output norm and gate fused into the store of o ("Kimi K3.1 Pro 架构完全拆解"
// §3.3): o <- sigmoid(gate) * weight * o / sqrt(mean(o^2) + eps) per
// (token, head) row over its dv channels.  gate: [T, H, dv] of o's element
// type; weight: [dv] fp32 or null (ones).
struct Epilogue {
  const void *gate = nullptr;
  const float *weight = nullptr;
  float eps = 1e-6f;
  bool on() const { return gate != nullptr; }
};

// Size of the fixed device scratch of the allocation-free prefill
// (kda_chunk_prefill_noalloc): its schedule tables, one per device.
constexpr size_t kNoAllocScratchBytes = 1u << 20;

// The device address of this device's fixed scratch (kda_scratch.hip):
// hipGetSymbolAddress on the first call per device, cached afterwards.
hipError_t noalloc_scratch(void **out);

// Launchers (enqueue only; return the hipGetLastError of the launch).
hipError_t launch_k1(int elt, const ChunkDesc *chunks, int32_t nchunks, int32_t H,
                     const void *q, const void *k, const void *g, const void *beta, void *ws,
                     const Prologue &pro, hipStream_t s);

// Chunk prep for bf16 inputs (the records launch_k1 writes for elt == 1).
hipError_t launch_prep_bf16(const ChunkDesc *chunks, int32_t nchunks, int32_t H, const void *q,
                            const void *k, const void *g, const void *beta, void *ws,
                            const Prologue &pro, hipStream_t s);

// mode 0: prefill/replay (width dv, writes o and exit states to final_a,
//         and the chains' state checkpoints to final_b when it is not null;
//         with the epilogue on, o leaves normalized and gated and the whole
//         dv-wide row is one workgroup's);
// mode 1: segment pass (width dk + dv: [S~ | M], no o; S~ to final_a, M to
//         final_b: m_scan_order 0 row-major, 1 at scan_m_index, 2 (bf16
//         records) as hi / lo bf16 at scan_m_bf16_index).
hipError_t launch_k2(int elt, int mode, const ChainDesc *chains, int32_t nchains, int32_t H,
                     const void *ws, const void *v, void *o, const float *init,
                     const float *sin, float *final_a, float *final_b, int m_scan_order,
                     const Epilogue &epi, hipStream_t s);

// Fused chunk prep + state chain, one workgroup per (chain, head) with all
// dv columns (bf16; entry states from `init` (init_idx >= 0), from the
// planner's `sin` (init_idx <= -2) or zero): writes o, exit states and (when
// ckpt is not null) the chains' state checkpoints; with the prologue and the
// output epilogue.
hipError_t launch_fused(const ChainDesc *chains, int32_t nchains, int32_t H, const void *q,
                         const void *k, const void *v, const void *g, const void *beta,
                         void *o, const float *init, const float *sin, float *final_state,
                         float *ckpt, hipStream_t s, const Prologue &pro = Prologue(),
                         const Epilogue &epi = Epilogue());

// The planner's first pass on the fused kernel (bf16), one launch: the
// first segment of every split sequence from its entry state (heads: o,
// checkpoints, exit state to head_final[final_idx]) beside the segment pass
// of its middle segments (segs: exit pair from [0 | I] with values [V | 0],
// S~ to st_out[final_idx] row-major and M to m_out[final_idx] as hi / lo
// bf16 at scan_m_bf16_index).
hipError_t launch_fused_pass1(const ChainDesc *heads, int32_t nheads, const ChainDesc *segs,
                              int32_t nsegs, int32_t H, const void *q, const void *k,
                              const void *v, const void *g, const void *beta, void *o,
                              const float *init, float *head_final, float *ckpt, float *st_out,
                              float *m_out, hipStream_t s, const Prologue &pro = Prologue(),
                              const Epilogue &epi = Epilogue());

// Whether the state chain's replay pass takes the output epilogue itself:
// when its plain launch runs 128-column blocks anyway (at least one wide
// workgroup per compute unit).  Otherwise it runs the 64-column blocks
// without it and launch_out_norm_gate follows.
bool k2_fuses_epilogue(int32_t nchains, int32_t H);

// The output norm and gate as a pass of its own over o ([rows, dv], in place).
hipError_t launch_out_norm_gate(int elt, int64_t rows, void *o, const Epilogue &epi,
                                hipStream_t s);

// elt 1 (bf16 planners): Mseg holds the hi / lo bf16 M of scan_m_bf16_index
// and the products run as three bf16 MFMAs; elt 0: fp32 M at scan_m_index.
hipError_t launch_scan(int elt, const ScanDesc *descs, int32_t ndesc, int32_t H, const float *Mseg,
                       const float *Stseg, const float *init, float *sin, hipStream_t s);

// The scan of one chain of nsteps row-major pairs (M [nsteps, H, dk, dk],
// S~ [nsteps, H, dk, dv]) from init ([H, dk, dv] or null: zero): writes the
// nsteps + 1 states sin[0] = init, sin[j + 1] = S~_j + M_j sin[j].
hipError_t launch_scan_rows(int32_t nsteps, int32_t H, const float *M, const float *St,
                            const float *init, float *sin, hipStream_t s);

// Speculative-decode replay: m accepted cached tokens, then P new tokens.
// The prologue applies to cached and new tokens, the epilogue to the new
// tokens' outputs.
hipError_t launch_replay(int elt, int32_t N, int32_t H, int32_t W, const int32_t *accepted,
                         const void *ck, const void *cv, const void *cg, const void *cb,
                         int32_t P, const void *q, const void *k, const void *v, const void *g,
                         const void *beta, float *state, void *o, const Prologue &pro,
                         const Epilogue &epi, hipStream_t s);

hipError_t launch_decode(int elt, int32_t N, int32_t H, const void *q, const void *k,
                         const void *v, const void *g, const void *beta, float *state, void *o,
                         const Prologue &pro, const Epilogue &epi, hipStream_t s);

} // namespace kda
