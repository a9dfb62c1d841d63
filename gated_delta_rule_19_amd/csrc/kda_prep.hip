// Chunk prep for bf16 inputs: the per-(chunk, head) record that the
// state-carrying kernel (kda_prefill.hip) consumes.
//
// The mathematics is the FlashKDA chunk form of "Kimi K3 的架構"
// (hao.cnyes.com) §六, with the 16-token reference points that the decay's
// lower bound allows ("Kimi K3.1 Pro 架构完全拆解" §3.2).  With G the
// inclusive cumulative log-decay from the chunk start, p_I = G before token
// tile I, G_loc = G - p_I and G_C the chunk total:
//   Q_loc = q e^{G_loc},  K_loc = k e^{G_loc},  K_st = k e^{-G_loc}
//   L_IJ  = Diag(beta) K_loc,I (K_st,J e^{p_I - p_J})^T  (J < I; strictly lower part of the diagonal tile)
//   M_IJ  = Q_loc,I (K_st,J e^{p_I - p_J})^T             (J < I; lower part incl. diagonal of the diagonal tile)
//   Q_decay = q e^{G},  K_decay = k e^{G},  K_restore = k e^{G_C - G},  a_last = e^{G_C}
//   INV Diag(beta) with INV = (I + L)^-1.
//
// Record, bf16 unless stated:
//   Q_decay [C][D], K_decay [C][D]        columns = channels
//   K_restore^T [D][C]                    row p = channel kperm(p), column kperm(token)
//   INV Diag(beta) [C][C], M_qk [C][C]    column kperm(token); lower triangular, so
//                                         only 6 of their 8 fragment blocks are stored
//   a_last [D] fp32                       entry p = channel kperm(p)
// The state kernel keeps channel kperm(p) in row p of its state, so each of
// these is an MFMA operand for it as stored.  The matrices are stored as
// their MFMA A fragments: 16-byte piece g of row r (8 consecutive row
// elements; G pieces per row, 16 or 8) sits at index
//   ((r / 16) * (G / 4) + g / 4) * 64 + (g % 4) * 16 + r % 16,
// so each 1 KiB block is the fragment of one 16-row tile and 32-column
// k-step, lane l's 16 bytes at 16 l.  The prep writes, the state kernel's
// copy into LDS and its fragment reads then all move 1 KiB of consecutive
// bytes per instruction.
//
// One workgroup of 4 waves per (chunk, head) item, persistent: workgroup b
// takes items b, b + grid, ..., two workgroups per compute unit.  Wave w
// owns token tile w: lane (lr, lg) = (lane % 16, lane / 16) holds token
// 16 w + lr and, for k-step s = 0..3, channels 32 s + 8 lg .. + 7 -- one
// 16-byte load or store per k-step, and the MFMA fragment layout.  Three
// stages per item, a barrier after the first two:
//   A  tile scan of g; Q_loc, K_loc, K_st; diagonal L and M_qk tiles; then
//      the loads of the item after next are issued
//   B  the previous item's INV Diag(beta) from LDS to its record; decay
//      factors; Q_decay, K_decay, M_qk to the record; K_restore^T to LDS;
//      off-diagonal L tiles to LDS; diagonal blocks of INV
//   C  K_restore^T to the record; off-diagonal blocks of INV, INV Diag(beta)
//      to LDS
// Stage A of the next item runs right after stage C, with no barrier between:
// A writes no region that C reads (beta is double-buffered by item parity).
//
// Transposed products keep the fragments of every result row-contiguous: an
// MFMA with its two operands swapped returns the transposed tile, in which a
// lane holds 4 consecutive columns of one row instead of 4 rows of one
// column; and K_restore^T is K_restore times a 0/1 selection matrix on the
// MFMA (exact: one nonzero term per output).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kPrepThreads = 256;
constexpr int kLdOp = kD + 8; // bf16 rows of 128 channels (272 B: a fragment's 16 rows start in distinct banks)
constexpr int kLdBk = 20;     // fp32 16 x 16 blocks (80-byte rows)
constexpr int kLdRt = kC + 8; // bf16 rows of 64 (144 B)
constexpr float kL2e = 1.4426950408889634f;

// record sections, in elements of their type
constexpr int kRecKd = kC * kD;          // bf16
constexpr int kRecKrT = 2 * kC * kD;     // bf16
constexpr int kRecInvb = 3 * kC * kD;    // bf16, the stored blocks of a triangular C x C
constexpr int kRecMqk = kRecInvb + kTriBlocks * 512; // bf16, likewise
constexpr int kRecAl = (kRecMqk + kTriBlocks * 512) / 2; // fp32
// An element offset past the end of every record: a store there falls
// outside the item's buffer resource and is dropped.  The pieces of a
// triangular section's unstored blocks go there, so that every path issues
// the same number of record stores.
constexpr int kRecDrop = 1 << 28;

// The 6 off-diagonal tile pairs (I, J), I > J, by wave: (3,0) (3,1) | (1,0) |
// (2,0) (2,1) | (3,2).  Each M_qk row piece that spans the tile pair
// (2m, 2m + 1) of one row tile then lies in a single wave, diagonal tiles
// (wave I) and zero tiles included, so M_qk goes out in 16-byte stores.
__host__ __device__ constexpr int prep_npairs(int w) { return (w == 0 || w == 2) ? 2 : 1; }
__host__ __device__ constexpr int prep_pair_I(int w) { return w == 0 ? 3 : w; }
__host__ __device__ constexpr int prep_pair_J(int w, int n) {
  return (w == 0 || w == 2) ? n : (w == 1 ? 0 : 2);
}
// index of the pair (I, J), I > J, among the 6
__host__ __device__ constexpr int offp(int I, int J) { return I * (I - 1) / 2 + J; }

struct PrepSmem {
  bf16 Kst[4][16][kLdOp];   // K_st per tile (stage A -> B)
  bf16 Aq3[2][16][kLdOp];   // K_loc, Q_loc of tile 3 (stage A -> B)
  float Tot[4][kD];         // per-tile totals of g (stage A -> B)
  float Beta[2][kC];        // beta, by item parity
  float Fac[4][3][kD];      // per tile: e^{p_I}, e^{tot_I}, e^{G_C - p_{I+1}} (wave-local)
  float Foff[6][kD];        // e^{p_I - p_J} of the off-diagonal pairs (wave-local)
  float Loff[6][16][kLdBk]; // off-diagonal blocks of L (stage B -> C)
  float Dinv[4][16][kLdBk]; // inverted diagonal blocks of I + L (stage B -> C)
  bf16 KrT[kD][kLdRt];      // K_restore^T staged in record layout (stage B -> C)
  bf16 Inv[kC][kLdRt];      // INV Diag(beta) staged (stage C -> next item's B)
};

// index of 16-byte piece g of row r in a piece-ordered section with G pieces
// per row
__host__ __device__ constexpr int piece_index(int r, int g, int G) {
  return ((r >> 4) * (G >> 2) + (g >> 2)) * 64 + (g & 3) * 16 + (r & 15);
}

// record element offset of the 16-byte piece g of row r (8 pieces per row)
// of the triangular section at `base`, or kRecDrop for a piece of one of its
// unstored blocks
__host__ __device__ constexpr int tri_piece(int base, int r, int g) {
  const int tb = tri_block(2 * (r >> 4) + (g >> 2));
  return tb < 0 ? kRecDrop : base + 8 * (tb * 64 + (g & 3) * 16 + (r & 15));
}

// Record stores go through one buffer resource per item (base address in
// scalar registers), each lane adding a 32-bit offset: a 64-bit address per
// lane and store would take two vector registers.  Offsets are in bf16
// elements.  The records are read only by the next kernel, so they are
// stored non-temporal (the whole 8192 x 96 call measured 0.605 -> 0.595 ms).
constexpr int kNt = 2; // cache-policy bits of a buffer access: nt
__device__ __forceinline__ void rec_store8(__amdgpu_buffer_rsrc_t r, int e, bf16x8 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, 2 * e, 0, kNt);
}
__device__ __forceinline__ void rec_store8(__amdgpu_buffer_rsrc_t r, int e, const f32x4 &lo,
                                           const f32x4 &hi) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = static_cast<bf16>(lo[i]);
    v[4 + i] = static_cast<bf16>(hi[i]);
  }
  rec_store8(r, e, v);
}

} // namespace

// PRO: the prologue (gate logits -> log decay, q / k L2 norm) is compiled in;
// which of its steps run is decided by A_log != null and qk_eps > 0.
template <bool PRO>
__global__ __launch_bounds__(kPrepThreads) __attribute__((amdgpu_waves_per_eu(2))) void prep_kernel(
    const ChunkDesc *__restrict__ chunks, int32_t H, const bf16 *__restrict__ q,
    const bf16 *__restrict__ k, const bf16 *__restrict__ g, const bf16 *__restrict__ beta,
    uint8_t *__restrict__ ws, int has_q, int32_t nitems, const float *__restrict__ A_log,
    float g_min, float qk_eps) {
  __shared__ __attribute__((aligned(16))) PrepSmem sm;
  const int pw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); // token tile
  const int64_t rowstride = (int64_t)H * kD;
  constexpr int64_t RB = (int64_t)k1_record_bytes(2);
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  // raw inputs of one item: this lane's token, channels 32 s + 8 lg .. + 7;
  // rows past the chunk end read 0 (no decay, no key, no query, beta 0).
  // beta stays raw until used: widening it at the load would make the wave
  // wait for every load in flight.
  // the blocks of INV Diag(beta) above the diagonal are zero and the
  // staging copy keeps them
  for (int e = threadIdx.x; e < 6 * 256; e += kPrepThreads) {
    const int t = e >> 8, rr = (e >> 4) & 15, c = e & 15;
    const int bi = t < 3 ? 0 : (t < 5 ? 1 : 2);
    const int bj = t < 3 ? t + 1 : (t < 5 ? t - 1 : 3);
    sm.Inv[16 * bi + rr][kperm(16 * bj + c)] = static_cast<bf16>(0.f);
  }

  u32x4 rg[4], rq[4], rk[4];
  unsigned short rbeta = 0;
  // prologue: the head's gate log scale, and whether this lane's token is
  // inside the chunk (rows past its end must not decay)
  const bool gate_on = PRO && A_log != nullptr, qk_on = PRO && qk_eps > 0.f;
  float rA = 0.f;
  bool rvalid = true;
  auto issue = [&](int item) {
    const int ln = opaque_lane(), lr = ln & 15, lg = ln >> 4, r = 16 * pw + lr;
    const int ci = item / H, h = item - ci * H;
    const ChunkDesc cd = chunks[ci];
    if (gate_on) {
      rA = A_log[h];
      rvalid = r < cd.len;
    }
    const int64_t base = cd.tok0 * rowstride + (int64_t)h * kD;
    const uint32_t nbytes = (uint32_t)(((cd.len - 1) * rowstride + kD) * 2);
    const __amdgpu_buffer_rsrc_t bg = buffer_rsrc(g + base, nbytes);
    const __amdgpu_buffer_rsrc_t bk = buffer_rsrc(k + base, nbytes);
    // without q the buffer is empty and every q load reads 0
    const __amdgpu_buffer_rsrc_t bq = buffer_rsrc(q + base, has_q ? nbytes : 0u);
    const __amdgpu_buffer_rsrc_t bb =
        buffer_rsrc(beta + cd.tok0 * H + h, (uint32_t)(((cd.len - 1) * (int64_t)H + 1) * 2));
    auto ld = [&](__amdgpu_buffer_rsrc_t b, int s) {
      const int vo = (int)((r * rowstride + 32 * s + 8 * lg) * 2);
      return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(b, vo, 0, 0));
    };
    // no branch around any of these loads: the number of memory operations
    // between them and their first use is then the same on every path, and
    // the wait for them does not also wait for this item's record stores
#pragma unroll
    for (int s = 0; s < 4; ++s)
      rg[s] = ld(bg, s);
    rbeta = __builtin_amdgcn_raw_buffer_load_b16(bb, (int)(r * H * 2), 0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      rk[s] = ld(bk, s);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      rq[s] = ld(bq, s);
  };

  // Q_loc, K_loc of this lane's token and channels as MFMA fragments (stage
  // A -> B; K_st goes through LDS)
  Frag<bf16> fq[4], fk[4];
  f32x4 accLc, accLr, accMr;

  // ---- stage A: tile scan, Q_loc / K_loc / K_st, diagonal tiles; then the
  // loads of item `next` (if any) ----------------------------------------------
  auto stage_a = [&](float *Bt, int next) {
    const int lane = opaque_lane(), lr = lane & 15, lg = lane >> 4, r = 16 * pw + lr;
    // inclusive cumulative sum over the tile's 16 tokens (one DPP row), then
    // the tile totals (lane 15 of each row) to LDS
    float G[4][8];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      widen8(rg[s], G[s]);
    if (gate_on) {
      const float ea = __builtin_amdgcn_exp2f(rA * kL2e);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          G[s][j] = rvalid ? gate_log_decay(G[s][j], ea, g_min) : 0.f;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        G[s][j] = row_scan16(G[s][j]);
    // prologue: 1 / |q|, 1 / |k| of this lane's token (its 128 channels are
    // spread over the four lanes lr, lr + 16, lr + 32, lr + 48)
    float iq = 1.f, ik = 1.f;
    if (qk_on) {
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sq = sumsq8_bf16(rq[s], sq);
        sk = sumsq8_bf16(rk[s], sk);
      }
      sq = add_xor32(add_xor16(sq));
      sk = add_xor32(add_xor16(sk));
      iq = __builtin_amdgcn_rsqf(sq + qk_eps);
      ik = __builtin_amdgcn_rsqf(sk + qk_eps);
    }
    if (lr == 15) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        *reinterpret_cast<f32x4 *>(&sm.Tot[pw][32 * s + 8 * lg]) =
            f32x4{G[s][0], G[s][1], G[s][2], G[s][3]};
        *reinterpret_cast<f32x4 *>(&sm.Tot[pw][32 * s + 8 * lg + 4]) =
            f32x4{G[s][4], G[s][5], G[s][6], G[s][7]};
      }
    }
    if (lg == 0)
      Bt[r] = __builtin_bit_cast(float, (unsigned)rbeta << 16);
    accLc = zero;
    accLr = zero;
    accMr = zero;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float qv[8], kv[8], xq[8], xk[8], xs[8];
      widen8(rq[s], qv);
      widen8(rk[s], kv);
      if (qk_on) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          qv[j] *= iq;
          kv[j] *= ik;
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = G[s][j] * kL2e;
        const float e1 = __builtin_amdgcn_exp2f(x);
        xq[j] = qv[j] * e1;
        xk[j] = kv[j] * e1;
        xs[j] = kv[j] * __builtin_amdgcn_exp2f(-x);
      }
      fq[s] = pack8(xq);
      fk[s] = pack8(xk);
      const Frag<bf16> fs = pack8(xs);
      *reinterpret_cast<bf16x8 *>(&sm.Kst[pw][lr][32 * s + 8 * lg]) = fs.v;
      if (pw == 3) {
        *reinterpret_cast<bf16x8 *>(&sm.Aq3[0][lr][32 * s + 8 * lg]) = fk[s].v;
        *reinterpret_cast<bf16x8 *>(&sm.Aq3[1][lr][32 * s + 8 * lg]) = fq[s].v;
      }
      // K_loc K_st^T in the column layout and its transpose, Q_loc K_st^T
      // transposed (row layout)
      mma(accLc, fk[s], fs);
      mma(accLr, fs, fk[s]);
      mma(accMr, fs, fq[s]);
    }
    // the raw inputs are consumed: the item after this one loads now and
    // has a whole item's time to arrive
    if (next < nitems)
      issue(next);
  };

  // Stage A of each item runs at the end of the previous item's iteration
  // (the first one before the loop), so the waits for its inputs never sit
  // at a loop-header merge, where they would be taken conservatively.
  int item = blockIdx.x, par = 0;
  if (item < nitems) {
    issue(item);
    stage_a(sm.Beta[0], item + gridDim.x);
  }
  // INV Diag(beta) of the previous item leaves its staging copy at the start
  // of the next item's stage B; before the first item the resource is empty,
  // so those stores are dropped (and every iteration stores the same number
  // of times)
  __amdgpu_buffer_rsrc_t prev = buffer_rsrc(ws, 0u);
  // piece u of a section with 8 pieces per row: row, first column
  auto piece_row = [](int u) { return 16 * (u >> 7) + (u & 15); };
  auto piece_col = [](int u) { return 8 * (4 * ((u >> 6) & 1) + ((u >> 4) & 3)); };
  auto inv_out = [&](__amdgpu_buffer_rsrc_t dst) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int u = (int)threadIdx.x + kPrepThreads * n;
      const int tb = tri_block(u >> 6);
      rec_store8(dst, tb < 0 ? kRecDrop : kRecInvb + 8 * (tb * 64 + (u & 63)),
                 *reinterpret_cast<const bf16x8 *>(&sm.Inv[piece_row(u)][piece_col(u)]));
    }
  };
  for (; item < nitems; item += gridDim.x, par ^= 1) {
    const __amdgpu_buffer_rsrc_t rr = buffer_rsrc(ws + (int64_t)item * RB, (uint32_t)RB);
    float *Bt = sm.Beta[par];
    lds_barrier();
    inv_out(prev);
    prev = rr;

    // ---- stage B ------------------------------------------------------------
    f32x4 y;  // this tile's diagonal block of INV, column layout
    f32x4 dv; // the same block times Diag(beta), row layout
    {
      const int lane = opaque_lane(), lr = lane & 15, lg = lane >> 4, r = 16 * pw + lr;
      {
        // this tile's factors for two channels per lane; the off-diagonal
        // pair factors of this wave's pairs; a_last (every wave stores the
        // same values, so the number of stores does not depend on the wave)
        const int c0 = 2 * lane;
        float t[4][2];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float2 x = *reinterpret_cast<const float2 *>(&sm.Tot[w][c0]);
          t[w][0] = x.x;
          t[w][1] = x.y;
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          float pI = 0.f, tI = 0.f, gc = 0.f;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            pI += w < pw ? t[w][e] : 0.f;
            tI += w == pw ? t[w][e] : 0.f;
            gc += t[w][e];
          }
          sm.Fac[pw][0][c0 + e] = __builtin_amdgcn_exp2f(pI * kL2e);             // <= 1
          sm.Fac[pw][1][c0 + e] = __builtin_amdgcn_exp2f(tI * kL2e);             // (e^-80, 1]
          sm.Fac[pw][2][c0 + e] = __builtin_amdgcn_exp2f((gc - pI - tI) * kL2e); // <= 1
#pragma unroll
          for (int n = 0; n < 2; ++n) {
            if (n < prep_npairs(pw)) {
              const int I = prep_pair_I(pw), J = prep_pair_J(pw, n);
              float sum = 0.f; // p_I - p_J = t_J + ... + t_{I-1} <= 0
#pragma unroll
              for (int w = 0; w < 3; ++w)
                sum += (w >= J && w < I) ? t[w][e] : 0.f;
              sm.Foff[offp(I, J)][c0 + e] = __builtin_amdgcn_exp2f(sum * kL2e);
            }
          }
          __builtin_amdgcn_raw_buffer_store_b32(
              __builtin_bit_cast(int, __builtin_amdgcn_exp2f(gc * kL2e)), rr,
              4 * (kRecAl + kperm_inv(c0 + e)), 0, 0);
        }
      }
      wave_lds_fence();
      // Q_decay and K_decay to the record, K_restore^T to its staging copy:
      //   Q_decay = Q_loc e^{p_I},  K_decay = K_loc e^{p_I},
      //   K_restore = (K_st e^{tot_I}) e^{G_C - p_{I+1}}
      // (K_st e^{tot_I} = k e^{p_{I+1} - G} <= |k|: every factor and partial
      // product is at most 1 in size, so a result underflows only where the
      // exact value is negligible).  K_restore^T comes from the selection
      // products: lane (n, lg) gets channel 32 s + 16 h + n of tokens
      // 16 pw + 4 lg .. + 3, which are 4 consecutive positions of its row.
      {
        // selection matrices: B operand h picks channels 16 h .. 16 h + 15
        // of a 32-channel k-step (lane (n, lg), element j: 1 where
        // 8 lg + j == 16 h + n); built from bit patterns, bf16 1.0 = 0x3f80
        Frag<bf16> sel[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int kk = 16 * h + lr - 8 * lg; // the element holding 1, if in 0..7
          const unsigned one = 0x3f80u << (16 * (kk & 1));
          u32x4 w;
#pragma unroll
          for (int d = 0; d < 4; ++d)
            w[d] = (kk >> 1) == d ? one : 0u;
          sel[h].v = __builtin_bit_cast(bf16x8, w);
        }
        const int kcol = 32 * (pw >> 1) + 8 * lg + 4 * (pw & 1);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          float f0[8], fe[8], fc[8], xq[8], xk[8], xs[8], yq[8], yk[8], yr[8];
          load8f(&sm.Fac[pw][0][32 * s + 8 * lg], f0);
          load8f(&sm.Fac[pw][1][32 * s + 8 * lg], fe);
          load8f(&sm.Fac[pw][2][32 * s + 8 * lg], fc);
          frag_to_f32(fq[s], xq);
          frag_to_f32(fk[s], xk);
          frag_to_f32(load_frag(&sm.Kst[pw][lr][32 * s + 8 * lg]), xs);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            yq[j] = xq[j] * f0[j];
            yk[j] = xk[j] * f0[j];
            yr[j] = (xs[j] * fe[j]) * fc[j];
          }
          const int pc = 8 * piece_index(r, 4 * s + lg, 16); // = 8 ((pw * 4 + s) * 64 + lane)
          rec_store8(rr, pc, pack8(yq).v);
          rec_store8(rr, kRecKd + pc, pack8(yk).v);
          const Frag<bf16> kr = pack8(yr);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            f32x4 t = zero;
            mma(t, kr, sel[h]);
            bf16x4 v4;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              v4[i] = static_cast<bf16>(t[i]);
            *reinterpret_cast<bf16x4 *>(&sm.KrT[kperm_inv(32 * s + 16 * h + lr)][kcol]) = v4;
          }
          // one k-step at a time: hoisting every step's LDS reads would
          // hold too many registers while the next item's loads are in flight
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // off-diagonal pairs (I, J): B = K_st of tile J times e^{p_I - p_J};
      // operands swapped, so the tiles come out in the row layout (lane:
      // row 16 I + lr, columns 16 J + 4 lg .. + 3)
      f32x4 accL[2], accM[2];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        accL[n] = zero;
        accM[n] = zero;
        if (n < prep_npairs(pw)) {
          const int I = prep_pair_I(pw), J = prep_pair_J(pw, n);
          const int pi = offp(I, J);
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const Frag<bf16> e = load_frag(&sm.Kst[J][lr][32 * s + 8 * lg]);
            float xs[8], fo[8];
            frag_to_f32(e, xs);
            load8f(&sm.Foff[pi][32 * s + 8 * lg], fo);
#pragma unroll
            for (int j = 0; j < 8; ++j)
              xs[j] *= fo[j];
            const Frag<bf16> b = pack8(xs);
            Frag<bf16> ak, aq;
            if (I == pw) {
              ak = fk[s];
              aq = fq[s];
            } else {
              ak = load_frag(&sm.Aq3[0][lr][32 * s + 8 * lg]);
              aq = load_frag(&sm.Aq3[1][lr][32 * s + 8 * lg]);
            }
            mma(accL[n], b, ak);
            mma(accM[n], b, aq);
          }
          *reinterpret_cast<f32x4 *>(&sm.Loff[pi][lr][4 * lg]) = accL[n] * Bt[16 * I + lr];
        }
      }

      // M_qk: the diagonal tile (lower incl. diagonal), the pairs and the
      // zero upper tiles; row piece (row tile I, column half m) = tiles
      // (I, 2m) | (I, 2m + 1), 8 record positions 32 m + 8 lg .. + 7
      {
        f32x4 md;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          md[i] = (4 * lg + i <= lr) ? accMr[i] : 0.f;
        auto put = [&](int I, int m, const f32x4 &lo, const f32x4 &hi) {
          rec_store8(rr, tri_piece(kRecMqk, 16 * I + lr, 4 * m + lg), lo, hi);
        };
        // two stores per wave on every path; the pieces of the unstored
        // all-zero blocks are dropped, and take their zeros from an opaque
        // value, so that no zero vector is hoisted out of the item loop and
        // kept in registers across it
        u32x4 zw;
        asm volatile("v_mov_b32 %0, 0\n\tv_mov_b32 %1, 0\n\tv_mov_b32 %2, 0\n\tv_mov_b32 %3, 0"
                     : "=v"(zw[0]), "=v"(zw[1]), "=v"(zw[2]), "=v"(zw[3]));
        const bf16x8 zz = __builtin_bit_cast(bf16x8, zw);
        if (pw == 0) {
          put(3, 0, accM[0], accM[1]);
          put(0, 0, md, zero);
        } else if (pw == 1) {
          put(1, 0, accM[0], md);
          rec_store8(rr, tri_piece(kRecMqk, 16 + lr, 4 + lg), zz); // unstored block: dropped
        } else if (pw == 2) {
          put(2, 0, accM[0], accM[1]);
          put(2, 1, md, zero);
        } else {
          put(3, 1, accM[0], md);
          rec_store8(rr, tri_piece(kRecMqk, lr, 4 + lg), zz); // unstored block: dropped
        }
      }

      // D^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8) for N = L of the diagonal
      // tile (N^16 = 0), with N and its powers in both layouts in registers
      const f32x4 bc = *reinterpret_cast<const f32x4 *>(&Bt[16 * pw + 4 * lg]);
      {
        const float br = Bt[16 * pw + lr];
        f32x4 nc, nr; // N[4 lg + i][lr], N[lr][4 lg + i]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          nc[i] = (lr < 4 * lg + i) ? bc[i] * accLc[i] : 0.f;
          nr[i] = (4 * lg + i < lr) ? br * accLr[i] : 0.f;
        }
        f32x4 n2c = zero, n2r = zero, n4c = zero, n4r = zero;
        mm16_rr(n2c, nr, nc);
        mm16_rr(n2r, nc, nr);
        mm16_rr(n4c, n2r, n2c);
        mm16_rr(n4r, n2c, n2r);
        y = zero;
        mm16_rr(y, n4r, n4c); // N^8
#pragma unroll
        for (int i = 0; i < 4; ++i)
          y[i] += (4 * lg + i == lr) ? 1.f : 0.f;
        mm16_rr(y, n4r, y);  // (I + N^4) Y
        mm16_rr(y, n2r, y);  // (I + N^2) Y
        mm16_rr(y, -nr, y);  // (I - N) Y
      }
      acc_store(&sm.Dinv[pw][0][0], kLdBk, y, lr, lg);
      wave_lds_fence();
      dv = *reinterpret_cast<const f32x4 *>(&sm.Dinv[pw][lr][4 * lg]) * bc;
    }
    lds_barrier();

    // ---- stage C: K_restore^T to the record; INV Diag(beta) to its staging
    // copy ---------------------------------------------------------------------
    {
      const int lane = opaque_lane(), lr = lane & 15, lg = lane >> 4;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int u = 64 * pw + lane + kPrepThreads * n;
        rec_store8(rr, kRecKrT + 8 * u,
                   *reinterpret_cast<const bf16x8 *>(&sm.KrT[piece_row(u)][piece_col(u)]));
      }
      // column block j = pw: dv on the diagonal, and below it the block
      // forward substitution X_ij = -D_i^-1 sum_{m=j}^{i-1} L_im X_mj, each
      // X_ij also formed in the row layout for its 8-byte piece of the
      // staging copy
      const int j = pw;
      f32x4 X[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        X[t] = (t == j) ? y : zero;
      const f32x4 bcj = *reinterpret_cast<const f32x4 *>(&Bt[16 * j + 4 * lg]);
      const int vcol = 32 * (j >> 1) + 8 * lg + 4 * (j & 1);
      auto put = [&](int i, const f32x4 &x) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v4[e] = static_cast<bf16>(x[e]);
        *reinterpret_cast<bf16x4 *>(&sm.Inv[16 * i + lr][vcol]) = v4;
      };
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i == j)
          put(i, dv);
        if (i > j) {
          f32x4 o = zero;
          f32x4 tsum = zero;
#pragma unroll
          for (int m = 0; m < 3; ++m)
            if (m >= j && m < i)
              mm16_lds_acc(tsum, &sm.Loff[offp(i, m)][0][0], kLdBk, X[m], lr, lg);
          const f32x4 nd = -*reinterpret_cast<const f32x4 *>(&sm.Dinv[i][lr][4 * lg]);
          if (i < 3) {
            f32x4 x = zero;
            mm16_rr(x, nd, tsum);
            X[i] = x;
          }
          mm16_rr(o, tsum, nd); // row layout
          put(i, o * bcj);
        }
      }
    }
    if (item + (int)gridDim.x < nitems)
      stage_a(sm.Beta[par ^ 1], item + 2 * (int)gridDim.x);
  }
  // the last item's INV Diag(beta)
  lds_barrier();
  inv_out(prev);
}

hipError_t launch_prep_bf16(const ChunkDesc *chunks, int32_t nchunks, int32_t H, const void *q,
                            const void *k, const void *g, const void *beta, void *ws,
                            const Prologue &pro, hipStream_t s) {
  if (nchunks == 0)
    return hipSuccess;
  // persistent grid: two workgroups per compute unit are resident (LDS)
  const int64_t nitems = (int64_t)nchunks * H;
  const int64_t resident = (int64_t)kComputeUnits * 2;
  dim3 grid((unsigned)std::min(nitems, resident)), block(kPrepThreads);
  // without q, k stands in as a readable buffer of the same shape
  const int has_q = q != nullptr;
  auto launch = [&](auto kern) {
    kern<<<grid, block, 0, s>>>(chunks, H, (const bf16 *)(has_q ? q : k), (const bf16 *)k,
                                (const bf16 *)g, (const bf16 *)beta, (uint8_t *)ws, has_q,
                                (int32_t)nitems, pro.A_log, pro.g_min, pro.qk_eps);
  };
  if (pro.on())
    launch(prep_kernel<true>);
  else
    launch(prep_kernel<false>);
  return hipGetLastError();
}

} // namespace kda
