// KDA chunked prefill on gfx950: chunk prep (K1), state-carrying chain (K2),
// and the sequence-split planner's prefix scan.
//
// The chunkwise form is the FlashKDA matrix form of "Kimi K3 的架構"
// (hao.cnyes.com), §六 FlashKDA 演算法: per chunk of C = 64 tokens and head,
//   a = exp(cumsum g),  K_decay = Diag(a) K,  Q_decay = Diag(a) Q,
//   K_inv = Diag(a)^-1 K,  K_restore = a[-1] * K_inv,
//   L = StrictTril(Diag(beta) K_decay K_inv^T),  INV = (I + L)^-1,
//   M_qk = tril(Q_decay K_inv^T)   (diagonal kept: an output reads the state
//                                    after its own token's update)
// and then, walking the chunks of a sequence in order,
//   U = INV Diag(beta) (V - K_decay S),  O = Q_decay S + M_qk U,
//   S = Diag(a[-1]) S + K_restore^T U.
//
// Numerics (the decay's lower bound, "Kimi K3.1 Pro 架构完全拆解" §3.2 and
// the orkas.ai page's section on that bound): a chunk-level K_inv would need
// exp(-cumsum g) up to e^320 and overflows fp32.  With g >= -5 every 16-token
// cumulative log-decay lies in (-80, 0], so the products exp(G_r - G_t) needed
// by L and M_qk are factored at 16-token reference points: with p_I the
// cumulative log-decay just before row tile I,
//     exp(G_r - G_t) = exp(G_r - p_I) * exp(p_I - G_t),
// the first factor in (e^-80, 1] for r in tile I, the second <= e^80 on the
// diagonal tile and <= 1 for earlier tiles.  Both fit bf16/fp32, so every
// 16 x 16 tile, the diagonal one included, is one dense MFMA product.
// Q_decay, K_decay and K_restore keep the chunk start/end as reference: their
// factors are <= 1 and underflow only where the exact value is negligible.
//
// INV is computed exactly (up to fp32 rounding) by blocked forward
// substitution over 16 x 16 blocks; any exact method gives the same unique
// inverse of the unit lower-triangular I + L.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kThreads = 256;

// Offsets inside one chunk-prep record (element size es).
struct RecOff {
  size_t qd, kd, krt, invb, mqk, ac;
  __host__ __device__ constexpr explicit RecOff(size_t es)
      : qd(0), kd(64 * 128 * es), krt(2 * 64 * 128 * es), invb(3 * 64 * 128 * es),
        mqk(3 * 64 * 128 * es + 64 * 64 * es), ac(3 * 64 * 128 * es + 2 * 64 * 64 * es) {}
};

// The 10 lower (row tile I, column tile J) pairs of a 64 x 64 chunk matrix,
// and the index of each off-diagonal pair among the 6 off-diagonal ones.
__device__ __constant__ int kPairI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__device__ __constant__ int kPairJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
__device__ __constant__ int kOffIdx[10] = {-1, 0, -1, 1, 2, -1, 3, 4, 5, -1};
// The 6 off-diagonal pairs (I > J) in the order of kOffIdx, and the 6 upper
// (I < J) tiles.
__device__ __constant__ int kOffI[6] = {1, 2, 2, 3, 3, 3};
__device__ __constant__ int kOffJ[6] = {0, 0, 1, 0, 1, 2};
__device__ __constant__ int kUpI[6] = {0, 0, 0, 1, 1, 2};
__device__ __constant__ int kUpJ[6] = {1, 2, 3, 2, 3, 3};


// 4 consecutive input elements kept as raw dwords between load and use.
template <typename T> struct Raw4;
template <> struct Raw4<bf16> {
  typedef unsigned int type __attribute__((ext_vector_type(2)));
  __device__ __forceinline__ static type load(__amdgpu_buffer_rsrc_t r, int voff) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
  }
  __device__ __forceinline__ static void widen(type w, float *x) {
    x[0] = __builtin_bit_cast(float, w[0] << 16);
    x[1] = __builtin_bit_cast(float, w[0] & 0xffff0000u);
    x[2] = __builtin_bit_cast(float, w[1] << 16);
    x[3] = __builtin_bit_cast(float, w[1] & 0xffff0000u);
  }
};
template <> struct Raw4<float> {
  typedef unsigned int type __attribute__((ext_vector_type(4)));
  __device__ __forceinline__ static type load(__amdgpu_buffer_rsrc_t r, int voff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
  }
  // (the whole vector is bit-cast: a bit-cast of one element of a vector
  // reads element 0 whatever the index with this compiler)
  __device__ __forceinline__ static void widen(type w, float *x) {
    const f32x4 v = __builtin_bit_cast(f32x4, w);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      x[j] = v[j];
  }
};

} // namespace

// ---------------------------------------------------------------------------
// K1: chunk prep, chunk-parallel.  A persistent grid: workgroup b handles
// (chunk, head) items b, b + grid, ..., and the inputs of its next item are
// loaded while the MFMA, inverse and store phases of the current one run.
// With has_q == 0 (segment transitions need no outputs) q is not a real
// input: Q_decay and M_qk are then 0.
//
// Thread t owns rows 4 (t / 16) .. + 3 of the chunk and the 8 channels that
// the record stores at positions 8 (t % 16) .. + 7 (kperm order: logical
// channels lc0 .. lc0 + 3 and lc0 + 16 .. lc0 + 19), so record rows go out
// as 16-byte stores.  Wave w holds exactly row tile w, so the 16-token
// reference points are sums of per-wave column totals.  The LDS operands of
// the L / M_qk products keep the same (permuted) channel order on both
// sides, which leaves the sums over channels unchanged.
// ---------------------------------------------------------------------------
// PRO: the prologue (gate logits -> log decay, q / k L2 norm) is compiled in;
// which of its steps run is decided by A_log != null and qk_eps > 0.
template <typename T, bool PRO>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void k1_kernel(
    const ChunkDesc *__restrict__ chunks, int32_t H, const T *__restrict__ q,
    const T *__restrict__ k, const T *__restrict__ g, const T *__restrict__ beta,
    uint8_t *__restrict__ ws, int has_q, int32_t nitems, const float *__restrict__ A_log,
    float g_min, float qk_eps) {
  constexpr int LD = kD + 16 / (int)sizeof(T); // operand row stride: rows 16 B apart in banks
  constexpr size_t OPB = (size_t)kC * LD * sizeof(T);
  constexpr RecOff off(sizeof(T));
  // Operand region: Q_loc, K_loc, K_start (3 x [C][LD] of T).  After the
  // MFMA phase it is reused for L (fp32), per-wave powers of its diagonal
  // block, the inverted diagonal blocks, and M_qk and INV Diag(beta) staged
  // in record layout.
  __shared__ __attribute__((aligned(16))) uint8_t smem[3 * OPB];
  __shared__ __attribute__((aligned(16))) float sWT[4][kD]; // per-wave totals of g
  __shared__ __attribute__((aligned(16))) float sF[6][kD];  // exp(p_I - p_J), I > J
  __shared__ float sBeta[kC];

  T(*sQl)[LD] = reinterpret_cast<T(*)[LD]>(smem);
  T(*sKl)[LD] = reinterpret_cast<T(*)[LD]>(smem + OPB);
  T(*sKs)[LD] = reinterpret_cast<T(*)[LD]>(smem + 2 * OPB);
  constexpr int LF = kC + 4;  // fp32 rows, 16-byte aligned
  constexpr int LB = 20;      // 16 x 16 fp32 blocks, 16-byte aligned rows
  constexpr int LM = kC + 16 / (int)sizeof(T);
  constexpr size_t POW0 = (size_t)kC * LF * 4;
  constexpr size_t DINV0 = POW0 + (size_t)4 * 2 * 16 * LB * 4;
  constexpr size_t MQ0 = DINV0 + (size_t)4 * 16 * LB * 4;
  constexpr size_t IB0 = MQ0 + (size_t)kC * LM * sizeof(T);
  float(*sL)[LF] = reinterpret_cast<float(*)[LF]>(smem);
  float(*sPow)[2][16][LB] = reinterpret_cast<float(*)[2][16][LB]>(smem + POW0);
  float(*sDinv)[16][LB] = reinterpret_cast<float(*)[16][LB]>(smem + DINV0);
  T(*sMq)[LM] = reinterpret_cast<T(*)[LM]>(smem + MQ0);
  T(*sIb)[LM] = reinterpret_cast<T(*)[LM]>(smem + IB0);
  static_assert(IB0 + (size_t)kC * LM * sizeof(T) <= 3 * OPB, "aliasing fits");

  const int tid = threadIdx.x;
  const int wv = tid >> 6, lane = tid & 63, lgp = lane >> 4;
  const int cg = tid & 15, row0 = 4 * (tid >> 4);
  const int lc0 = 32 * (cg >> 2) + 4 * (cg & 3);
  const int64_t rowstride = (int64_t)H * kD;
  // logical channel of this thread's e-th record position
  auto lch = [&](int e) { return e < 4 ? lc0 + e : lc0 + 12 + e; };

  // raw inputs of one item: 4 rows x (2 runs of 4 channels) of g, k, q, and
  // beta of row tid (tid < C); buffers over rows 0..len-1 of the (chunk,
  // head), so rows past the chunk end read 0 (no decay, no key, no query)
  using Raw = typename Raw4<T>::type;
  Raw rwg[4][2], rwk[4][2], rwq[4][2];
  float rbeta = 0.f;
  auto issue_loads = [&](int item) {
    const int ci = item / H, h = item - ci * H;
    const ChunkDesc cd = chunks[ci];
    const int64_t base = cd.tok0 * rowstride + (int64_t)h * kD;
    const uint32_t nbytes = (uint32_t)(((cd.len - 1) * rowstride + kD) * sizeof(T));
    const __amdgpu_buffer_rsrc_t rg = buffer_rsrc(g + base, nbytes);
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(k + base, nbytes);
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(q + base, nbytes);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int vo = (int)(((row0 + j) * rowstride + lc0 + 16 * u) * sizeof(T));
        rwg[j][u] = Raw4<T>::load(rg, vo);
        rwk[j][u] = Raw4<T>::load(rk, vo);
        if (has_q)
          rwq[j][u] = Raw4<T>::load(rq, vo);
      }
    if (tid < kC) {
      const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(
          beta + cd.tok0 * H + h, (uint32_t)(((cd.len - 1) * (int64_t)H + 1) * sizeof(T)));
      rbeta = buffer_load1(rb, (int)(tid * H * (int)sizeof(T)), beta);
    }
  };

  if ((int)blockIdx.x < nitems)
    issue_loads(blockIdx.x);
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
  const int ci = item / H, h = item - ci * H;
  const ChunkDesc cd = chunks[ci];
  const int len = cd.len;
  uint8_t *rec = ws + ((int64_t)ci * H + h) * k1_record_bytes(sizeof(T));
  T *Qd = reinterpret_cast<T *>(rec + off.qd);
  T *Kd = reinterpret_cast<T *>(rec + off.kd);
  T *KrT = reinterpret_cast<T *>(rec + off.krt);
  T *INVb = reinterpret_cast<T *>(rec + off.invb);
  T *Mqk = reinterpret_cast<T *>(rec + off.mqk);
  float *ac = reinterpret_cast<float *>(rec + off.ac);

  lds_barrier(); // the previous item's last LDS reads are done
  // g is widened now; k and q stay raw until their row is used (registers)
  float gv[4][8];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int u = 0; u < 2; ++u)
      Raw4<T>::widen(rwg[j][u], &gv[j][4 * u]);
  if (tid < kC)
    sBeta[tid] = rbeta;
  // prologue: the log decay from the gate logits (rows past the chunk end
  // decay by nothing), and 1 / |q|, 1 / |k| per row (a row's 128 channels
  // are spread over 16 consecutive lanes, channel group t % 16)
  float iq[4] = {1.f, 1.f, 1.f, 1.f}, ik[4] = {1.f, 1.f, 1.f, 1.f};
  if constexpr (PRO) {
    if (A_log != nullptr) {
      const float ea = __expf(A_log[h]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          gv[j][e] = row0 + j < len ? g_min / (1.f + __expf(-ea * gv[j][e])) : 0.f;
    }
    if (qk_eps > 0.f) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float a[4], b[4];
          Raw4<T>::widen(rwk[j][u], b);
          if (has_q)
            Raw4<T>::widen(rwq[j][u], a);
          else
            a[0] = a[1] = a[2] = a[3] = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sq += a[e] * a[e];
            sk += b[e] * b[e];
          }
        }
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) {
          sq += __shfl_xor(sq, m);
          sk += __shfl_xor(sk, m);
        }
        iq[j] = 1.f / __builtin_sqrtf(sq + qk_eps);
        ik[j] = 1.f / __builtin_sqrtf(sk + qk_eps);
      }
    }
  }

  // ---- phase 1: inclusive cumulative log-decay per channel -------------
  // own rows, then the 4 row groups of the wave (lanes 16 apart), then the
  // waves before this one (per-wave totals through LDS)
  float G[4][8], ex[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float run = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      run += gv[j][e];
      G[j][e] = run;
    }
    float x = run;
    float y = __shfl_up(x, 16);
    if (lgp >= 1)
      x += y;
    y = __shfl_up(x, 32);
    if (lgp >= 2)
      x += y;
    ex[e] = x - run;
    if (lgp == 3)
      sWT[wv][8 * cg + e] = x;
  }
  lds_barrier();
  // p_own = p_wv (before this tile), p_next = p_{wv+1}, p_last = G_last
  float pown[8], pnext[8], plast[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    pown[e] = 0.f;
    pnext[e] = 0.f;
    plast[e] = 0.f;
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const f32x4 t0 = *reinterpret_cast<const f32x4 *>(&sWT[w][8 * cg]);
    const f32x4 t1 = *reinterpret_cast<const f32x4 *>(&sWT[w][8 * cg + 4]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float t = e < 4 ? t0[e] : t1[e - 4];
      if (w < wv)
        pown[e] += t;
      if (w <= wv)
        pnext[e] += t;
      plast[e] += t;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      G[j][e] += pown[e] + ex[e];

  // off-diagonal factors exp(p_I - p_J) for the 6 tile pairs I > J, pair
  // p = row group p (I = 1,2,2,3,3,3; J = 0,0,1,0,1,2): the B operand of pair
  // (I, J) is K_start of tile J times this factor, k_t exp(p_I - G_t) <= 1
  {
    const int p = tid >> 4;
    if (p < 6) {
      const int I = p < 1 ? 1 : (p < 3 ? 2 : 3);
      const int J = p - I * (I - 1) / 2;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        x[e] = 0.f;
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        // w < I adds into p_I, w < J subtracts p_J
        const f32x4 t0 = *reinterpret_cast<const f32x4 *>(&sWT[w][8 * cg]);
        const f32x4 t1 = *reinterpret_cast<const f32x4 *>(&sWT[w][8 * cg + 4]);
        const float sgn = (w < I ? 1.f : 0.f) - (w < J ? 1.f : 0.f);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          x[e] += sgn * (e < 4 ? t0[e] : t1[e - 4]);
      }
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        f[e] = __expf(x[e]);
      *reinterpret_cast<f32x4 *>(&sF[p][8 * cg]) = f32x4{f[0], f[1], f[2], f[3]};
      *reinterpret_cast<f32x4 *>(&sF[p][8 * cg + 4]) = f32x4{f[4], f[5], f[6], f[7]};
    }
  }
  if (tid < 16) { // a_last per logical channel
    float a[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      a[e] = __expf(plast[e]);
    store4(ac + lc0, a[0], a[1], a[2], a[3]);
    store4(ac + lc0 + 16, a[4], a[5], a[6], a[7]);
  }

  // ---- phase 2: decayed operands ----------------------------------------
  // two passes, one per run of 4 channels (fewer live registers), each
  // writing 8-byte pieces of the record rows and LDS operand rows
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    float eP[4], eR[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      eP[e] = __expf(pown[4 * u + e]);                   // exp(p_I)            <= 1
      eR[e] = __expf(plast[4 * u + e] - pnext[4 * u + e]); // exp(G_last - p_I+1) <= 1
    }
    float kr[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = row0 + j;
      float kv[4], qv[4];
      Raw4<T>::widen(rwk[j][u], kv);
      if (has_q)
        Raw4<T>::widen(rwq[j][u], qv);
      else
        qv[0] = qv[1] = qv[2] = qv[3] = 0.f;
      if constexpr (PRO) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qv[e] *= iq[j];
          kv[e] *= ik[j];
        }
      }
      float xq[4], xk[4], xs[4], xQ[4], xK[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float Gv = G[j][4 * u + e], po = pown[4 * u + e];
        const float eloc = __expf(Gv - po);                 // (e^-80, 1]
        const float est = __expf(po - Gv);                  // [1, e^80)
        const float eend = __expf(pnext[4 * u + e] - Gv);   // (e^-80, 1]
        xq[e] = qv[e] * eloc;
        xk[e] = kv[e] * eloc;
        xs[e] = kv[e] * est;
        const float ga = eloc * eP[e]; // exp(G_r)
        xQ[e] = qv[e] * ga;
        xK[e] = kv[e] * ga;
        kr[e][j] = kv[e] * (eend * eR[e]); // exp(G_last - G_r) k
      }
      const int pc = 8 * cg + 4 * u; // record / operand position of channel run u
      store4(&sQl[r][pc], xq[0], xq[1], xq[2], xq[3]);
      store4(&sKl[r][pc], xk[0], xk[1], xk[2], xk[3]);
      store4(&sKs[r][pc], xs[0], xs[1], xs[2], xs[3]);
      store4(Qd + r * kD + pc, xQ[0], xQ[1], xQ[2], xQ[3]);
      store4(Kd + r * kD + pc, xK[0], xK[1], xK[2], xK[3]);
    }
    // K_restore^T: row = logical channel, this thread's 4 tokens are
    // contiguous under kperm
#pragma unroll
    for (int e = 0; e < 4; ++e)
      store4(KrT + lch(4 * u + e) * kC + kperm(row0), kr[e][0], kr[e][1], kr[e][2], kr[e][3]);
  }
  lds_barrier();

  // ---- phase 3: L and M_qk tiles on MFMA ---------------------------------
  const int lr = lane & 15, lg = lane >> 4;
  f32x4 accL[3], accM[3];
#pragma unroll
  for (int pp = 0; pp < 3; ++pp) {
    accL[pp] = f32x4{0.f, 0.f, 0.f, 0.f};
    accM[pp] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int p = wv + 4 * pp;
    if (p < 10) {
      const int I = kPairI[p], J = kPairJ[p];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kb = 32 * s + 8 * lg;
        const Frag<T> aK = load_frag(&sKl[16 * I + lr][kb]);
        const Frag<T> aQ = load_frag(&sQl[16 * I + lr][kb]);
        Frag<T> b;
        if (I == J) {
          b = load_frag(&sKs[16 * J + lr][kb]);
        } else {
          const Frag<T> e = load_frag(&sKs[16 * J + lr][kb]);
          float x[8];
          frag_to_f32(e, x);
          const float *f = &sF[kOffIdx[p]][kb];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            x[j] *= f[j];
          b = frag_from_f32<T>(x);
        }
        mma(accL[pp], aK, b);
        mma(accM[pp], aQ, b);
      }
    }
  }
  lds_barrier(); // operand region is now free for L / INV

  // L (beta-scaled rows, strictly lower) and M_qk (lower incl. diagonal, in
  // record layout) to LDS.
#pragma unroll
  for (int pp = 0; pp < 3; ++pp) {
    const int p = wv + 4 * pp;
    if (p < 10) {
      const int I = kPairI[p], J = kPairJ[p];
      const int col = 16 * J + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * I + 4 * lg + i;
        sL[row][col] = (col < row) ? sBeta[row] * accL[pp][i] : 0.f;
        sMq[row][kperm(col)] = from_f32<T>((col <= row) ? accM[pp][i] : 0.f);
      }
    }
  }
  // zero the upper tiles (J > I) of M_qk and INV Diag(beta)
  for (int e = tid; e < 6 * 256; e += kThreads) {
    const int t = e >> 8, r = (e >> 4) & 15, cc = e & 15;
    const int row = 16 * kUpI[t] + r, col = 16 * kUpJ[t] + cc;
    sMq[row][kperm(col)] = from_f32<T>(0.f);
    sIb[row][kperm(col)] = from_f32<T>(0.f);
  }
  lds_barrier();

  // the next item's inputs are in flight during the rest of this one
  if (item + (int)gridDim.x < nitems)
    issue_loads(item + gridDim.x);

  // ---- phase 4: INV = (I + L)^-1 by 16 x 16 blocks on fp32 MFMA ----------
  // Level 0 (wave b): D_b = I + N with N = L_bb strictly lower, so
  // D_b^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8) exactly (N^16 = 0).
  // Level 1 (wave j): block forward substitution down column block j,
  // X_ij = -D_i^-1 sum_{m=j}^{i-1} L_im X_mj, from its own earlier blocks,
  // L and the D_i^-1 of level 0.  Blocks stay in accumulator layout
  // (lane (lr, lg) holds rows 4 lg .. + 3 of column lr), which is also a
  // valid B operand, so each product feeds the next.
  {
    const int lr = lane & 15, lg = lane >> 4;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 X[4];
    // INV Diag(beta) block (I, J) into the staged record layout
    auto put = [&](int I, int J, const f32x4 &x) {
      const float bcol = sBeta[16 * J + lr];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sIb[16 * I + 4 * lg + i][kperm(16 * J + lr)] = from_f32<T>(x[i] * bcol);
    };
    {
      const int b = wv;
      const float *N = &sL[16 * b][16 * b];
      float *P2 = &sPow[b][0][0][0];
      float *P4 = &sPow[b][1][0][0];
      const f32x4 n1 = acc_load(N, LF, lr, lg);
      f32x4 n2 = zero, n4 = zero, y = zero;
      mm16_lds_acc(n2, N, LF, n1, lr, lg); // N^2
      acc_store(P2, LB, n2, lr, lg);
      mm16_lds_acc(n4, P2, LB, n2, lr, lg); // N^4
      acc_store(P4, LB, n4, lr, lg);
      mm16_lds_acc(y, P4, LB, n4, lr, lg); // N^8
#pragma unroll
      for (int i = 0; i < 4; ++i)
        y[i] += (4 * lg + i == lr) ? 1.f : 0.f; // I + N^8
      mm16_lds_acc(y, P4, LB, y, lr, lg);       // (I + N^4) Y
      mm16_lds_acc(y, P2, LB, y, lr, lg);       // (I + N^2) Y
      mm16_lds_acc(y, N, LF, y, lr, lg, -1.f);  // (I - N) Y
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (t == b)
          X[t] = y; // static register index
      acc_store(&sDinv[b][0][0], LB, y, lr, lg);
      put(b, b, y);
    }
    lds_barrier(); // every D_i^-1 is in LDS
    {
      const int j = wv;
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        if (i > j) {
          f32x4 t = zero;
#pragma unroll
          for (int m = 0; m < 3; ++m)
            if (m >= j && m < i)
              mm16_lds_acc(t, &sL[16 * i][16 * m], LF, X[m], lr, lg);
          f32x4 x = zero;
          mm16_lds_acc(x, &sDinv[i][0][0], LB, t, lr, lg, -1.f);
          X[i] = x;
          put(i, j, x);
        }
      }
    }
  }
  lds_barrier();

  // M_qk and INV Diag(beta) from their staging blocks to the record, 16
  // bytes per store
  {
    constexpr int UPR = kC * (int)sizeof(T) / 16; // 16-byte units per row
    constexpr int EPU = 16 / (int)sizeof(T);      // elements per unit
#pragma unroll
    for (int u = tid; u < kC * UPR; u += kThreads) {
      const int row = u / UPR, c0 = (u % UPR) * EPU;
      *reinterpret_cast<uint4 *>(Mqk + row * kC + c0) =
          *reinterpret_cast<const uint4 *>(&sMq[row][c0]);
      *reinterpret_cast<uint4 *>(INVb + row * kC + c0) =
          *reinterpret_cast<const uint4 *>(&sIb[row][c0]);
    }
  }
  } // item loop
}

// ---------------------------------------------------------------------------
// K2: state-carrying chain.  One workgroup per (chain, head, column block of
// BV = 128 or 64 state columns); wave w owns the NCT 16-column tiles
// starting at vcol0 + 16 NCT w, so one workgroup reads each chunk
// record once for its BV columns, and each A fragment a wave reads from LDS
// serves all of its column tiles.
// The columns of V, U, O and S are independent, so each wave carries its own
// 128-row slice of S through the chunks with no exchange: the state, W, U
// and O stay in MFMA accumulators, and each accumulator feeds the next
// product as its B operand directly (the record's A operands are stored in
// kperm column order to match).  The chunk records are copied into LDS once
// per workgroup (double-buffered: chunk i+1's record is in flight while
// chunk i is computed), so the only barrier is one per chunk.
//   MODE 0: prefill / replay, width dv; writes o and the exit state (out_a)
//           and, for chains that hold one, the state checkpoint (out_b).
//   MODE 1: segment pass, width dk + dv of [S~ | M] from [0 | I] with values
//           [V | 0]; the exit state's S~ part goes to out_a, M part to out_b.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ Frag<T> pack_acc_pair(const f32x4 &lo, const f32x4 &hi) {
  const float x[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return frag_from_f32<T>(x);
}

// LDS image of a chunk record.  fp32 records: the same sections, each row
// padded by 16 bytes so that the 16 rows one wave reads per MFMA fragment
// start in different LDS banks (a 256- or 128-byte row stride would put
// them all in the same banks).  bf16 records are stored as 1 KiB fragment
// blocks (block (tile, k-step) holds the 16-byte fragment of lane l at
// 16 l) and the image is the record itself: a fragment read is 64
// consecutive 16-byte pieces.
template <typename T> struct RecLds {
  static constexpr bool pieces = false;
  static constexpr int es = sizeof(T);
  static constexpr int rowD = kD * es, rowC = kC * es;     // global row bytes
  static constexpr int padD = rowD + 16, padC = rowC + 16; // LDS row bytes
  static constexpr int qd = 0;
  static constexpr int kd = qd + kC * padD;
  static constexpr int krt = kd + kC * padD;
  static constexpr int invb = krt + kD * padC;
  static constexpr int mqk = invb + kC * padC;
  static constexpr int ac = mqk + kC * padC;
  static constexpr int bytes = ac + kD * 4;
  static constexpr int blocks = (bytes + 1023) / 1024;
};
template <> struct RecLds<bf16> {
  static constexpr bool pieces = true;
  static constexpr int qd = 0;
  static constexpr int kd = qd + kC * kD * 2;
  static constexpr int krt = kd + kC * kD * 2;
  static constexpr int invb = krt + kD * kC * 2;
  static constexpr int mqk = invb + kTriBlocks * 1024; // stored blocks only (tri_block)
  static constexpr int ac = mqk + kTriBlocks * 1024;
  static constexpr int bytes = ac + kD * 4;
  static constexpr int blocks = (bytes + 1023) / 1024;
};

// Gather offset inside one padded section: LDS byte q of a section with
// PAD-byte rows holds record byte base_g + r ROW + c (r = q / PAD, c = q % PAD);
// padding bytes (c >= ROW) read record byte 0.
template <int PAD, int ROW>
__device__ __forceinline__ int section_src(int q, int base_g) {
  const int r = q / PAD, c = q - r * PAD;
  return c < ROW ? base_g + r * ROW + c : 0;
}


// Copy of one chunk record (global) into its padded LDS image with
// direct-to-LDS loads: wave w fills 1 KiB blocks w, w + NW, ...; lane l of a
// block writes LDS bytes 16 l .. 16 l + 15, gathered from wherever they live
// in the record.  Every section of the image starts on a 1 KiB boundary, so
// a block lies in one section, chosen by a wave-uniform branch.  Completion
// is awaited with vmcnt(0).
template <typename T, int NW> struct RecordCopy {
  using L = RecLds<T>;
  static_assert(L::kd % 1024 == 0 && L::krt % 1024 == 0 && L::invb % 1024 == 0 &&
                    L::mqk % 1024 == 0 && L::ac % 1024 == 0,
                "sections must start on 1 KiB blocks");
  static constexpr int kPerWave = (L::blocks + NW - 1) / NW;
  // This lane's record byte offset for each of its wave's blocks; the same
  // for every chunk, so it is computed once per workgroup.
  __device__ __forceinline__ static void offsets(int (&goff)[kPerWave], int wv, int lane) {
    constexpr int RB = (int)k1_record_bytes(sizeof(T));
    if constexpr (L::pieces) { // the image is the record
#pragma unroll
      for (int j = 0; j < kPerWave; ++j) {
        const int p = (wv + j * NW) * 1024 + lane * 16;
        goff[j] = p < RB ? p : 0;
      }
    } else {
      constexpr RecOff off(sizeof(T));
#pragma unroll
      for (int j = 0; j < kPerWave; ++j) {
        const int b = wv + j * NW; // wave-uniform
        const int p = b * 1024 + lane * 16;
        int g = 0;
        if (b >= L::blocks)
          g = 0;
        else if (b * 1024 < L::kd)
          g = section_src<L::padD, L::rowD>(p - L::qd, (int)off.qd);
        else if (b * 1024 < L::krt)
          g = section_src<L::padD, L::rowD>(p - L::kd, (int)off.kd);
        else if (b * 1024 < L::invb)
          g = section_src<L::padC, L::rowC>(p - L::krt, (int)off.krt);
        else if (b * 1024 < L::mqk)
          g = section_src<L::padC, L::rowC>(p - L::invb, (int)off.invb);
        else if (b * 1024 < L::ac)
          g = section_src<L::padC, L::rowC>(p - L::mqk, (int)off.mqk);
        else
          g = p - L::ac < kD * 4 ? (int)off.ac + (p - L::ac) : 0;
        goff[j] = g;
      }
    }
  }
  __device__ __forceinline__ static void issue(uint8_t *lds, const uint8_t *src,
                                               const int (&goff)[kPerWave], int wv) {
    issue_part<0, 1>(lds, src, goff, wv);
  }
  // Part P of NP of this wave's blocks (the copy spread over a phase's
  // products, so that the wave's instruction issue never waits behind a
  // burst of copies)
  template <int P, int NP>
  __device__ __forceinline__ static void issue_part(uint8_t *lds, const uint8_t *src,
                                                    const int (&goff)[kPerWave], int wv) {
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(src, (uint32_t)k1_record_bytes(sizeof(T)));
#pragma unroll
    for (int j = P * kPerWave / NP; j < (P + 1) * kPerWave / NP; ++j) {
      const int b = wv + j * NW; // wave-uniform
      if (b >= L::blocks)
        break;
      lds_load16(r, goff[j], lds + b * 1024);
    }
  }
};

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// EPI: o leaves through the output norm and gate (mode 0, whole rows: the
// workgroup carries all dv columns).
template <typename T, int MODE, int BV, int NCT, int NBUF, bool EPI>
__global__ __launch_bounds__(k2_threads(BV, NCT)) void k2_kernel(
    const ChainDesc *__restrict__ chains, int32_t npairs, int32_t H,
    const uint8_t *__restrict__ ws, const T *__restrict__ v, T *__restrict__ o,
    const float *__restrict__ init, const float *__restrict__ sin, float *__restrict__ out_a,
    float *__restrict__ out_b, int32_t m_scan_order, const T *__restrict__ ogate,
    const float *__restrict__ onw, float oeps) {
  static_assert(!EPI || (MODE == 0 && BV == kD), "the output norm needs whole rows");
  constexpr int NW = k2_threads(BV, NCT) / 64;
  using L = RecLds<T>;
  constexpr int RB = (int)k1_record_bytes(sizeof(T));
  constexpr int RBP = L::blocks * 1024; // LDS image, whole 1 KiB blocks
  static_assert(NBUF == 1 || 2 * RBP <= 160 * 1024, "two record buffers must fit in LDS");
  // fragment addressing: padded images take the row length (elements) of
  // 128- and 64-wide rows, fragment-block images the k-steps per row
  constexpr int LD = L::pieces ? kD / 32 : RecLds<float>::padD / 4;
  constexpr int LC = L::pieces ? kC / 32 : RecLds<float>::padC / 4;
  __shared__ __attribute__((aligned(1024))) uint8_t srecA[RBP];
  __shared__ __attribute__((aligned(1024))) uint8_t srecB[NBUF == 2 ? RBP : 1];
  // bf16: each wave's own 64 x VW slice of the chunk's v also goes through
  // LDS (direct-to-LDS loads, 16 bytes per lane); fp32 keeps it in registers
  // (its record leaves no room).
  constexpr bool VLDS = sizeof(T) == 2;
  constexpr int VW = 16 * NCT;
  __shared__ __attribute__((aligned(16))) T sv[VLDS ? NW : 1][VLDS ? kC * VW : 1];
  // bf16 o of up to 4 waves leaves through a per-wave LDS tile: the
  // accumulator layout holds 4 rows of one column per lane, so direct stores
  // are 16 two-byte stores per lane; the tile read back row-wise is two
  // 16-byte stores (the 8-wave block has no LDS left for it).  The tile of
  // chunk ch is written to LDS in chunk ch and leaves at the start of chunk
  // ch + 1, after the barrier that waited for the next record's copy: any
  // memory operation of this wave while that copy is in flight waits for it
  // (a store behind the copy's instructions, an LDS read for its possible
  // aliasing), which cost a sixth of the chunk step.
  constexpr bool OT = VLDS && MODE == 0 && NW <= 4 && NCT == 1 && !EPI;
  __shared__ __attribute__((aligned(16))) T sot[OT ? NW : 1][OT ? kC * VW : 1];
  // output norm: per-wave partial sums of squares of each token row, and each
  // wave's own copy of the rows' scale factors
  __shared__ __attribute__((aligned(16))) float sRed[EPI ? NW : 1][EPI ? kC : 1];
  __shared__ __attribute__((aligned(16))) float sScl[EPI ? NW : 1][EPI ? kC : 1];

  // Workgroup -> (chain, head, column block): the column blocks of one
  // (chain, head) pair are 8 workgroups apart, so they run on the same XCD
  // (workgroups go to the 8 XCDs round-robin) at about the same time, and
  // all but the first read each chunk record from that XCD's L2.
  constexpr int NCB = (MODE == 1 ? 2 * kD : kD) / BV;
  const int grp = blockIdx.x / (8 * NCB), rem = blockIdx.x - grp * 8 * NCB;
  const int pair = 8 * grp + (rem & 7);
  if (pair >= npairs)
    return;
  const int chain_i = pair / H, h = pair - chain_i * H;
  const ChainDesc cd = chains[chain_i];
  const int col0 = (rem >> 3) * BV;
  const bool mpart = (MODE == 1) && (col0 >= kD);
  const int vcol0 = mpart ? col0 - kD : col0;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wcol = vcol0 + 16 * NCT * wv + lr; // this lane's column in tile c: wcol + 16c
  const int64_t rowstride = (int64_t)H * kD;
  const int nch = (cd.ntok + kC - 1) / kC;

  // S[c][ct]: rows 16 ct + 4 lg + i (ct = 0..7), column wcol + 16 c.  Row p
  // holds channel srow(p): the channel itself for fp32 records, kperm(p)
  // for bf16 ones (whose K_decay / Q_decay columns are in channel order).
  constexpr bool kPermRows = sizeof(T) == 2;
  auto srow = [](int p) { return kPermRows ? kperm(p) : p; };
  f32x4 S[NCT][8];
  {
    const float *ip = nullptr;
    if (MODE == 0) {
      if (cd.init_idx >= 0)
        ip = init + ((int64_t)cd.init_idx * H + h) * (kD * kD);
      else if (cd.init_idx <= -2)
        ip = sin + ((int64_t)(-2 - cd.init_idx) * H + h) * (kD * kD);
    }
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * ct + 4 * lg + i, col = wcol + 16 * c;
          S[c][ct][i] = ip ? ip[srow(row) * kD + col] : ((mpart && srow(row) == col) ? 1.f : 0.f);
        }
  }

  if (nch > 0) {
    const uint8_t *rec0 = ws + ((int64_t)cd.chunk0 * H + h) * RB;
    const int64_t rec_step = (int64_t)H * RB;
    const T *vchain = v + cd.tok0 * rowstride + (int64_t)h * kD + wcol;
    // v of one chunk for this lane: rows 16 tt + 4 lg + i (clamped into the
    // chunk), column wcol + 16 c
    auto load_v = [&](T (&dst)[NCT][4][4], int chunk) {
      const int len = min(kC, cd.ntok - chunk * kC);
      const T *vb = vchain + (int64_t)chunk * kC * rowstride;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const T *vr = vb + (int64_t)min(16 * tt + 4 * lg + i, len - 1) * rowstride;
#pragma unroll
          for (int c = 0; c < NCT; ++c)
            dst[c][tt][i] = vr[16 * c];
        }
    };
    // bf16 path: rows 0..63 of this wave's VW columns of one chunk into its
    // LDS slice; lane l of instruction j moves 16 bytes (8 columns) of row
    // (64 j + l) / (2 NCT); rows past the chunk end read as 0
    auto v_to_lds = [&](int chunk) {
      if constexpr (VLDS) {
        if (mpart)
          return;
        const int clen = min(kC, cd.ntok - chunk * kC);
        const T *vb = v + (cd.tok0 + (int64_t)chunk * kC) * rowstride + (int64_t)h * kD +
                      vcol0 + VW * wv;
        const __amdgpu_buffer_rsrc_t rv =
            buffer_rsrc(vb, (uint32_t)((clen - 1) * rowstride + VW) * sizeof(T));
#pragma unroll
        for (int j = 0; j < 2 * NCT; ++j) {
          const int u = 64 * j + lane, r = u / (2 * NCT), q = u % (2 * NCT);
          lds_load16(rv, (int)((r * rowstride + 8 * q) * sizeof(T)),
                     reinterpret_cast<uint8_t *>(&sv[wv][0]) + 1024 * j);
        }
      }
    };
    using RCopy = RecordCopy<T, NW>;
    int goff[RCopy::kPerWave];
    RCopy::offsets(goff, wv, lane);
    RCopy::issue(srecA, rec0, goff, wv);
    T vcur[VLDS ? 1 : NCT][4][4];
    if constexpr (VLDS)
      v_to_lds(0);
    else
      load_v(vcur, 0);
    wait_vmem();
    __syncthreads();

    // Output norm and gate of one chunk's O tile ("Kimi K3.1 Pro 架构完全拆解"
    // §3.3): O[r][c] <- sigmoid(gate) w[c] O[r][c] / sqrt(mean_c O[r][c]^2 + eps).
    // Lane (lr, lg) holds rows 16 tt + 4 lg + i of columns wcol + 16 c.  The
    // sums of squares are reduce-scattered over the 16 lanes of a row group
    // (lane lr ends with row tt = lr / 4, i = lr % 4), summed over the waves
    // through LDS (one barrier), and every wave keeps its own copy of the 64
    // scale factors.
    [[maybe_unused]] float wnorm[NCT];
    if constexpr (EPI) {
#pragma unroll
      for (int c = 0; c < NCT; ++c)
        wnorm[c] = onw ? onw[wcol + 16 * c] : 1.f;
    }
    [[maybe_unused]] auto norm_gate = [&](f32x4 (&Oa)[NCT][4], T (&gt)[EPI ? NCT : 1][4][4],
                                          int64_t tok, int len) {
      if constexpr (!VLDS) {
        const T *gb = ogate + tok * rowstride + (int64_t)h * kD + wcol;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const T *gr = gb + (int64_t)min(16 * tt + 4 * lg + i, len - 1) * rowstride;
#pragma unroll
            for (int c = 0; c < NCT; ++c)
              gt[c][tt][i] = gr[16 * c];
          }
      }
      float x[16];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float a = 0.f;
#pragma unroll
          for (int c = 0; c < NCT; ++c)
            a += Oa[c][tt][i] * Oa[c][tt][i];
          x[4 * tt + i] = a;
        }
#pragma unroll
      for (int st = 8; st >= 1; st >>= 1) {
        const bool up = (lr & st) != 0;
#pragma unroll
        for (int m = 0; m < st; ++m) {
          const float send = up ? x[m] : x[m + st];
          const float keep = up ? x[m + st] : x[m];
          x[m] = keep + __shfl_xor(send, st);
        }
      }
      sRed[wv][16 * (lr >> 2) + 4 * lg + (lr & 3)] = x[0];
      __syncthreads();
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w)
        tot += sRed[w][lane];
      sScl[wv][lane] = __builtin_amdgcn_rsqf(tot * (1.f / kD) + oeps);
      wave_lds_fence();
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const f32x4 sc = *reinterpret_cast<const f32x4 *>(&sScl[wv][16 * tt + 4 * lg]);
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float z = to_f32(gt[c][tt][i]);
            const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
            Oa[c][tt][i] *= sc[i] * wnorm[c] * sg;
          }
      }
    };

    // the chain's next checkpoint chunk and its index (wave-uniform)
    [[maybe_unused]] int ck_next = cd.ckpt_chunk, ck_idx = cd.ckpt_idx;

    // o of chunk ch from this wave's LDS tile (OT): row lane / 2 (+ 32),
    // columns 8 (lane % 2) .. + 7; rows past the chunk end fall outside the
    // buffer and are dropped
    [[maybe_unused]] auto flush_o = [&](int ch) {
      if constexpr (OT) {
        const int len = min(kC, cd.ntok - ch * kC);
        const int64_t tok = cd.tok0 + (int64_t)ch * kC;
        const __amdgpu_buffer_rsrc_t ro =
            buffer_rsrc(o + tok * rowstride + (int64_t)h * kD,
                        (uint32_t)((len - 1) * rowstride + kD) * sizeof(T));
        const T *ot = &sot[wv][0];
        const int ln = opaque_lane();
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int r = 32 * j + (ln >> 1), c8 = 8 * (ln & 1);
          const bf16x8 x = *reinterpret_cast<const bf16x8 *>(&ot[r * VW + c8]);
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(u32x4, x), ro,
              (int)((r * rowstride + vcol0 + VW * wv + c8) * sizeof(T)), 0, 0);
        }
      }
    };

    // One chunk: computes from the record image in `cur` while chunk ch+1's
    // record goes into `nxt`.  The buffers are distinct LDS objects and the
    // loop is unrolled by two, so every access names its buffer statically
    // and the compiler does not make reads of `cur` wait for the copy.
    auto chunk_step = [&](const int ch, uint8_t *cur, uint8_t *nxt)
                          __attribute__((always_inline)) {
      if constexpr (OT) {
        if (ch > 0)
          flush_o(ch - 1);
      }
      const int len = min(kC, cd.ntok - ch * kC);
      const int64_t tok = cd.tok0 + (int64_t)ch * kC;
      const bool more = ch + 1 < nch;
      // chunk ch+1: its record straight into the other LDS buffer (fp32:
      // its v into registers); in flight while chunk ch is computed
      T vnxt[VLDS ? 1 : NCT][4][4];
      // bf16: output gate logits of this chunk, first of all: the wait for
      // them at the store of o then covers none of the loads below (fp32
      // loads them at the store: its registers are full)
      T gt[EPI ? NCT : 1][4][4];
      if constexpr (EPI && VLDS) {
        const T *gb = ogate + tok * rowstride + (int64_t)h * kD + wcol;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const T *gr = gb + (int64_t)min(16 * tt + 4 * lg + i, len - 1) * rowstride;
#pragma unroll
            for (int c = 0; c < NCT; ++c)
              gt[c][tt][i] = gr[16 * c];
          }
      }
      // (v first: a wait the compiler places before these register loads
      // must not cover the record copy)
      if (more) {
        if constexpr (!VLDS)
          load_v(vnxt, ch + 1);
      }
      __builtin_amdgcn_sched_barrier(0); // keep the loads issued here, ahead of the math
      // (the record copy of chunk ch+1 is issued in four parts over the
      // first phase's k-steps below)
      const uint8_t *rec_nxt = rec0 + (int64_t)(ch + 1) * rec_step;

      const uint8_t *R = cur;
      const T *Qd = reinterpret_cast<const T *>(R + L::qd);
      const T *Kd = reinterpret_cast<const T *>(R + L::kd);
      const T *KrT = reinterpret_cast<const T *>(R + L::krt);
      const T *INVb = reinterpret_cast<const T *>(R + L::invb);
      const T *Mqk = reinterpret_cast<const T *>(R + L::mqk);
      const float *ac = reinterpret_cast<const float *>(R + L::ac);

      // Every product runs its k-steps in the outer loop, so the 4 to 8
      // accumulators of a step are independent MFMAs, and the A fragments of
      // the next step (or phase) are read from LDS before the current step's
      // MFMAs are issued.
      auto frag = [&](const T *base, int ld, int tile, int s) {
        if constexpr (L::pieces)
          return load_frag(base + ((tile * ld + s) * 64 + lane) * 8);
        else
          return load_frag(base + (16 * tile + lr) * ld + 32 * s + 8 * lg);
      };
      // INV Diag(beta) and M_qk are lower triangular: their blocks (row
      // tile 0 or 1, tokens 32..63) are zero, not stored in bf16 records and
      // not multiplied
      auto frag_tri = [&](const T *base, int tile, int s) {
        if constexpr (L::pieces)
          return load_frag(base + (tri_block(2 * tile + s) * 64 + lane) * 8);
        else
          return frag(base, LC, tile, s);
      };

      // W = K_decay S, O = Q_decay S (K = channels, B operand = S)
      Frag<T> bs[NCT][4];
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          bs[c][s] = pack_acc_pair<T>(S[c][2 * s], S[c][2 * s + 1]);
      f32x4 W[NCT][4], Oa[NCT][4];
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          W[c][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
          Oa[c][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      Frag<T> ak[4], aq[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        ak[tt] = frag(Kd, LD, tt, 0);
        if (MODE == 0)
          aq[tt] = frag(Qd, LD, tt, 0);
      }
      Frag<T> ai[2][4]; // INV Diag(beta) fragments, read during the last step
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (NBUF == 2 && more) {
          if (s == 0)
            RCopy::template issue_part<0, 4>(nxt, rec_nxt, goff, wv);
          else if (s == 1)
            RCopy::template issue_part<1, 4>(nxt, rec_nxt, goff, wv);
          else if (s == 2)
            RCopy::template issue_part<2, 4>(nxt, rec_nxt, goff, wv);
          else
            RCopy::template issue_part<3, 4>(nxt, rec_nxt, goff, wv);
        }
        Frag<T> nk[4], nq[4];
        if (s < 3) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            nk[tt] = frag(Kd, LD, tt, s + 1);
            if (MODE == 0)
              nq[tt] = frag(Qd, LD, tt, s + 1);
          }
        } else {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            ai[0][tt] = frag_tri(INVb, tt, 0);
            if (tt >= 2)
              ai[1][tt] = frag_tri(INVb, tt, 1);
          }
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int c = 0; c < NCT; ++c) {
            mma(W[c][tt], ak[tt], bs[c][s]);
            if (MODE == 0)
              mma(Oa[c][tt], aq[tt], bs[c][s]);
          }
        if (s < 3) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            ak[tt] = nk[tt];
            aq[tt] = nq[tt];
          }
        }
      }
      // V - W, then U = INV Diag(beta) (V - W)  (K = tokens)
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * tt + 4 * lg + i;
            // (bf16: rows past the chunk end were loaded as 0; fp32 loads
            // clamp the row and are masked here)
            float vv;
            if constexpr (VLDS)
              vv = mpart ? 0.f : to_f32(sv[wv][row * VW + 16 * c + lr]);
            else
              vv = (!mpart && row < len) ? to_f32(vcur[c][tt][i]) : 0.f;
            W[c][tt][i] = vv - W[c][tt][i];
          }
      // bf16: this wave's slice of v is consumed; chunk ch+1's goes in now
      if constexpr (VLDS) {
        if (more) {
          __builtin_amdgcn_s_waitcnt(0xc07f); // lgkmcnt(0): the slice reads have returned
          v_to_lds(ch + 1);
        }
      }
      Frag<T> bw[NCT][2];
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          bw[c][s] = pack_acc_pair<T>(W[c][2 * s], W[c][2 * s + 1]);
      Frag<T> am[2][4]; // M_qk fragments, read while U is computed
      if (MODE == 0) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          am[0][tt] = frag_tri(Mqk, tt, 0);
          if (tt >= 2)
            am[1][tt] = frag_tri(Mqk, tt, 1);
        }
      }
      f32x4 U[NCT][4];
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          U[c][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int tt = s == 1 ? 2 : 0; tt < 4; ++tt)
#pragma unroll
          for (int c = 0; c < NCT; ++c)
            mma(U[c][tt], ai[s][tt], bw[c][s]);
      Frag<T> bu[NCT][2];
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          bu[c][s] = pack_acc_pair<T>(U[c][2 * s], U[c][2 * s + 1]);
      // K_restore^T fragments of the first half of the state update, read
      // while O is finished
      Frag<T> ar[2][4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        ar[0][ct] = frag(KrT, LC, ct, 0);
        ar[1][ct] = frag(KrT, LC, ct, 1);
      }
      // O = Q_decay S + M_qk U
      if (MODE == 0) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int tt = s == 1 ? 2 : 0; tt < 4; ++tt)
#pragma unroll
            for (int c = 0; c < NCT; ++c)
              mma(Oa[c][tt], am[s][tt], bu[c][s]);
        if constexpr (EPI)
          norm_gate(Oa, gt, tok, len);
        // rows past the chunk end fall outside the buffer and are dropped
        const __amdgpu_buffer_rsrc_t ro =
            buffer_rsrc(o + tok * rowstride + (int64_t)h * kD,
                        (uint32_t)((len - 1) * rowstride + kD) * sizeof(T));
        if constexpr (OT) {
          // tile row 16 tt + 4 lg + i, column lr (flush_o at the start of
          // the next chunk, or after the last)
          T *ot = &sot[wv][0];
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              ot[(16 * tt + 4 * lg + i) * VW + lr] = from_f32<T>(Oa[0][tt][i]);
        } else {
          const int vo = (int)((4 * lg * rowstride + wcol) * sizeof(T));
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int so = (int)((16 * tt + i) * rowstride * sizeof(T)); // wave-uniform
#pragma unroll
              for (int c = 0; c < NCT; ++c)
                buffer_store(ro, from_f32<T>(Oa[c][tt][i]), vo + 16 * c * (int)sizeof(T), so);
            }
        }
      }
      // S = Diag(a_last) S + K_restore^T U, in two halves of 4 row tiles
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        Frag<T> nr[2][4];
        if (hf == 0) {
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            nr[0][ct] = frag(KrT, LC, ct + 4, 0);
            nr[1][ct] = frag(KrT, LC, ct + 4, 1);
          }
        }
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const f32x4 a4 = *reinterpret_cast<const f32x4 *>(ac + 16 * (4 * hf + ct) + 4 * lg);
#pragma unroll
          for (int c = 0; c < NCT; ++c)
            S[c][4 * hf + ct] *= a4;
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int c = 0; c < NCT; ++c)
              mma(S[c][4 * hf + ct], ar[s][ct], bu[c][s]);
        if (hf == 0) {
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            ar[0][ct] = nr[0][ct];
            ar[1][ct] = nr[1][ct];
          }
        }
      }
      // prefill: the state after this chunk is also a checkpoint (out_b);
      // its addresses come from an opaque lane index, so that they are
      // formed here and not kept in registers across the chunk loop
      if (MODE == 0 && out_b != nullptr && ch == ck_next && ch <= cd.ckpt_last) {
        const int ln = opaque_lane(), clg = ln >> 4;
        float *cp = out_b + ((int64_t)ck_idx * H + h) * (kD * kD) + vcol0 +
                    16 * NCT * wv + (ln & 15);
        ck_next += cd.ckpt_every;
        ++ck_idx;
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
          for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              cp[srow(16 * ct + 4 * clg + i) * kD + 16 * c] = S[c][ct][i];
      }

      if (more) {
        if (NBUF == 1) {
          __syncthreads(); // every wave is done with the record
          RCopy::issue(cur, rec0 + (int64_t)(ch + 1) * rec_step, goff, wv);
        }
        wait_vmem();
        __syncthreads();
        if constexpr (!VLDS) {
#pragma unroll
          for (int c = 0; c < NCT; ++c)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                vcur[c][tt][i] = vnxt[c][tt][i];
        }
      }
    };
    if constexpr (NBUF == 2) {
      for (int ch = 0; ch < nch; ch += 2) {
        chunk_step(ch, srecA, srecB);
        if (ch + 1 < nch)
          chunk_step(ch + 1, srecB, srecA);
      }
    } else {
      for (int ch = 0; ch < nch; ++ch)
        chunk_step(ch, srecA, srecA);
    }
    if constexpr (OT)
      flush_o(nch - 1);
  }

  float *fp = nullptr;
  if (cd.final_idx >= 0) {
    float *base = (MODE == 1 && mpart) ? out_b : out_a;
    fp = base + ((int64_t)cd.final_idx * H + h) * (kD * kD);
  }
  if (fp) {
    const int order = (MODE == 1 && mpart) ? m_scan_order : 0;
    if (order == 2) { // hi / lo bf16 for the bf16 scan
      bf16 *fb = reinterpret_cast<bf16 *>(fp);
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = srow(16 * ct + 4 * lg + i), col = wcol + 16 * c;
            const int x = scan_m_bf16_index(r, col);
            const bf16 hi = static_cast<bf16>(S[c][ct][i]);
            fb[x] = hi;
            fb[kD * kD + x] = static_cast<bf16>(S[c][ct][i] - static_cast<float>(hi));
          }
    } else {
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = srow(16 * ct + 4 * lg + i), col = wcol + 16 * c;
            fp[order == 1 ? scan_m_index(r, col) : r * kD + col] = S[c][ct][i];
          }
    }
  }
}

// ---------------------------------------------------------------------------
// Planner scan: entry states of the segments of one split sequence,
//   Sin[0] = S_0,   Sin[j+1] = S~_j + M_j Sin[j]
// ("部署 Kimi K3：从 KDA Kernel 到 Fleet 调度", §二: S = S~ + M S_in, pairs
// compose associatively).  Serial over segments, parallel over heads and
// column blocks of kScanBV = 16 state columns, fp32 throughout (fp32 calls
// and kda_segment_scan; bf16 calls use scan_bf16_kernel below).
//
// One workgroup of four waves per (sequence, head, column block).  Each step
// is a 128 x 16 x 128 product on v_mfma_f32_16x16x4f32: wave w owns output
// rows 32w .. 32w + 31 (two 16-row tiles) and all 128 reduction indices.  The
// k-step (i, e) of a lane in lane group kq = lane / 16 reduces over state row
//   m = 16 i + 4 kq + e     (i = 0..7, e = 0..3),
// so the lane's A operand is four consecutive reduction indices of M_j per i
// (M_j is stored in that order, scan_m_index: one 16-byte load per lane and
// 1 KiB contiguous per wave) and its B operand four contiguous floats of the
// transposed state in LDS.  The loads of M_{j+1} and S~_{j+1} are spread
// over step j's products, and the state goes through LDS (double-buffered,
// one barrier per step).
// ---------------------------------------------------------------------------
namespace {

struct ScanIn {
  f32x4 a[8][2]; // a[i][t][e] = M[32w + 16t + lane % 16][16 i + 4 kq + e]
  float st[2][4]; // st[t][e] = S~[32w + 16t + 4 kq + e][col0 + lane % 16]
  float warm[2];  // L2 warm-up loads of a later step (values unused)
};

constexpr int kScanLd = kD + 4; // LDS row stride (floats) of the transposed state

} // namespace

//
// ROWS: M_j is row-major (M[r][m] at r * dk + m), as kda_segment_transition
// writes it; the lane's four consecutive reduction indices are then one
// 16-byte load from its own row.  descs == null: the one sequence `one`.
template <bool ROWS>
__global__ __launch_bounds__(kThreads) void scan_kernel(const ScanDesc *__restrict__ descs,
                                                        ScanDesc one, int32_t ndesc, int32_t H,
                                                        const float *__restrict__ Mseg,
                                                        const float *__restrict__ Stseg,
                                                        const float *__restrict__ init,
                                                        float *__restrict__ sin) {
  static_assert(kScanBV == 16 && kThreads == 256, "thread map assumes 16 columns, 4 waves");
  constexpr int NCB = kD / kScanBV;
  // Column blocks of one (sequence, head) sit 8 workgroup ids apart, so they
  // run on one XCD and share its L2 copy of M_j and S~_j.
  const int grp = blockIdx.x / (8 * NCB), rem = blockIdx.x - grp * 8 * NCB;
  const int pair = 8 * grp + (rem & 7);
  if (pair >= ndesc * H)
    return;
  const int di = pair / H, h = pair - di * H;
  const ScanDesc d = descs ? descs[di] : one;
  const int col0 = (rem >> 3) * kScanBV;

  __shared__ __attribute__((aligned(16))) float sT[2][kScanBV][kScanLd]; // [buf][col][row]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, kq = lane >> 4;
  const int64_t mat = (int64_t)kD * kD;

  // entry state of segment 0: init (or zero) -> LDS and Sin[sin0]
  {
    const int m = tid >> 1, c0 = (tid & 1) * 8;
    f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = x0;
    if (d.init_idx >= 0) {
      const float *src = init + ((int64_t)d.init_idx * H + h) * mat + m * kD + col0 + c0;
      x0 = *reinterpret_cast<const f32x4 *>(src);
      x1 = *reinterpret_cast<const f32x4 *>(src + 4);
    }
    float *dst = sin + ((int64_t)d.sin0 * H + h) * mat + m * kD + col0 + c0;
    *reinterpret_cast<f32x4 *>(dst) = x0;
    *reinterpret_cast<f32x4 *>(dst + 4) = x1;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      sT[0][c0 + c][m] = x0[c];
      sT[0][c0 + 4 + c][m] = x1[c];
    }
  }

  const int nstep = d.nseg - 1;
  const int cb = rem >> 3;
  // Loads of step j in the order the products consume them.  The two warm-up
  // loads touch step j + 1's lines of M (this column block's eighth) and of
  // S~ (this block's columns), so that step's own loads, issued one step
  // later, hit L2.
  auto mat_at = [&](const float *base, int j) {
    return base + ((int64_t)(d.pair0 + j) * H + h) * mat;
  };
  // the rest of step j's inputs: S~ and the two warm-up loads, which touch
  // step j + 1's lines of M (this column block's eighth) and of S~ (this
  // block's columns) so that its own loads, issued a step later, hit L2
  auto load_rest = [&](ScanIn &in, int j) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float *sr = mat_at(Stseg, j) + (32 * w + 16 * t + 4 * kq) * kD + col0 + n;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        in.st[t][e] = sr[e * kD];
    }
    const int jw = min(j + 1, nstep - 1);
    in.warm[0] = mat_at(Mseg, jw)[(cb * 64 + lane) * 32];
    in.warm[1] = mat_at(Stseg, jw)[(tid & 127) * kD + col0];
  };
  // the A operands of k-group i, row tile t: 1 KiB block (8 w + i) * 2 + t
  // in scan order, else M[32 w + 16 t + n][16 i + 4 kq .. + 3]
  auto load_a = [&](ScanIn &in, const float *mj, int i) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
      in.a[i][t] = *reinterpret_cast<const f32x4 *>(
          ROWS ? mj + (32 * w + 16 * t + n) * kD + 16 * i + 4 * kq
               : mj + ((8 * w + i) * 2 + t) * 256 + 4 * lane);
  };
  auto load = [&](ScanIn &in, int j) {
    const float *mj = mat_at(Mseg, j);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      load_a(in, mj, i);
    load_rest(in, j);
  };
  // step j: reads sT[j & 1], writes sT[(j + 1) & 1] and Sin[sin0 + j + 1];
  // loads the inputs of step j + 1 (clamped: the last step reloads its own)
  auto step = [&](const ScanIn &cur, ScanIn &nxt, int j) {
    const int jn = min(j + 1, nstep - 1);
    const float *mn = mat_at(Mseg, jn);
    const float *src = &sT[j & 1][n][4 * kq];
    f32x4 b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      b[i] = *reinterpret_cast<const f32x4 *>(src + 16 * i);
    load_rest(nxt, jn);
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      load_a(nxt, mn, i);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(cur.a[i][t][e], b[i][e], acc[t], 0, 0, 0);
    }
    // issue order: the B reads, the S~ and warm-up loads of step j + 1, then
    // two of its M loads per eight products
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 10, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
    // the warm-up values are consumed (as nothing) only here, a step after
    // their loads were issued
    asm volatile("" ::"v"(cur.warm[0]), "v"(cur.warm[1]));
    float *dst = sin + ((int64_t)(d.sin0 + j + 1) * H + h) * mat + col0 + n;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[t][e] += cur.st[t][e];
      const int r0 = 32 * w + 16 * t + 4 * kq;
      *reinterpret_cast<f32x4 *>(&sT[(j + 1) & 1][n][r0]) = acc[t];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dst[(r0 + e) * kD] = acc[t][e];
    }
    __syncthreads();
  };

  ScanIn in0, in1;
  if (nstep > 0) // (no pairs: only the entry state is written)
    load(in0, 0);
  __syncthreads();
  int j = 0;
  for (; j + 2 <= nstep; j += 2) {
    step(in0, in1, j);
    step(in1, in0, j + 1);
  }
  if (j < nstep)
    step(in0, in1, j);
}

// ---------------------------------------------------------------------------
// The planner scan of bf16 calls.  Same recurrence, grid and state handling
// as scan_kernel; the product M_j Sin[j] runs on v_mfma_f32_16x16x32_bf16.
// M = M_hi + M_lo as the segment pass writes it (scan_m_bf16_index), and the
// state is split into three bf16 parts x = x_hi + x_mid + x_lo, exactly (each
// part takes the next 8 significant bits).  Then
//   M S ~= M_hi (S_hi + S_mid + S_lo) + M_lo S_hi,
// four bf16 MFMAs (16 cycles each) per 32-wide k-step in place of eight fp32
// ones (32 cycles each).  The terms left out, M_lo (S_mid + S_lo) and the
// remainder of M below M_lo, are of relative size 2^-16 of the product, far
// below the bf16 rounding of the chain's own products; M = I (no decay, no
// writes) carries the state exactly.  Sums and the state stay fp32: the
// thread that forms an entry of the next state splits it once into its
// LDS copy, where the B operands are read.  With the products this cheap a
// step is bound by the latency of its M loads, so the workgroup has 8
// compute waves (16 state rows each, 32 VGPRs of M per lane and step) that
// keep three steps' inputs in registers, each loaded two steps before its
// use, and a ninth wave that warms L2 with the lines of later steps.  Its
// loads sit in its own in-order memory counter: warm-up loads issued by the
// compute waves themselves lengthened their waits (101 against 72 us for 63
// steps of 12 heads).
// ---------------------------------------------------------------------------
namespace {

constexpr int kScanBf16Threads = 576; // 8 waves: wave w owns state rows 16 w .. + 15; wave 8 warms L2
constexpr int kScanBf16Ahead = 2;     // steps between a load of M_j and its use
constexpr int kScanBf16Warm = 3;      // steps between wave 8's L2 warm-up of a step and its use

struct ScanInBf16 {
  bf16x8 a[4][2]; // a[s][p]: part p (hi, lo) of M[16w + lane % 16][32 s + 8 kq .. + 7]
  float st[4];    // st[e] = S~[16w + 4 kq + e][col0 + lane % 16]
};

constexpr int kScanLdB = kD + 8; // LDS row stride (bf16) of a transposed state part

// x = hi + mid + lo exactly, each part bf16 (round to nearest)
__device__ __forceinline__ void split3(float x, bf16 &hi, bf16 &mid, bf16 &lo) {
  hi = static_cast<bf16>(x);
  const float r = x - static_cast<float>(hi);
  mid = static_cast<bf16>(r);
  lo = static_cast<bf16>(r - static_cast<float>(mid));
}

} // namespace

__global__ __launch_bounds__(kScanBf16Threads) void scan_bf16_kernel(
    const ScanDesc *__restrict__ descs, int32_t ndesc, int32_t H, const bf16 *__restrict__ Mseg,
    const float *__restrict__ Stseg, const float *__restrict__ init, float *__restrict__ sin) {
  static_assert(kScanBV == 16, "thread map assumes 16 columns");
  constexpr int NCB = kD / kScanBV;
  // column blocks of one (sequence, head) 8 workgroup ids apart: one XCD
  const int grp = blockIdx.x / (8 * NCB), rem = blockIdx.x - grp * 8 * NCB;
  const int pair = 8 * grp + (rem & 7);
  if (pair >= ndesc * H)
    return;
  const int di = pair / H, h = pair - di * H;
  const ScanDesc d = descs[di];
  const int col0 = (rem >> 3) * kScanBV;

  // the state's three parts, transposed: [buf][part][col][row]
  __shared__ __attribute__((aligned(16))) bf16 sB[2][3][kScanBV][kScanLdB];
  __shared__ __attribute__((aligned(16))) float sWarm[64]; // wave 8's loads land here, unread
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, kq = lane >> 4;
  const int64_t mat = (int64_t)kD * kD;

  // entry state of segment 0: init (or zero) -> LDS and Sin[sin0], or
  // Sin[sin0] as it stands -> LDS
  if (w < 8) {
    const int m = tid >> 2, c0 = (tid & 3) * 4;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    float *s0 = sin + ((int64_t)d.sin0 * H + h) * mat + m * kD + col0 + c0;
    if (d.init_idx == kScanEntryInSin)
      x = *reinterpret_cast<const f32x4 *>(s0);
    else {
      if (d.init_idx >= 0)
        x = *reinterpret_cast<const f32x4 *>(init + ((int64_t)d.init_idx * H + h) * mat +
                                             m * kD + col0 + c0);
      *reinterpret_cast<f32x4 *>(s0) = x;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16 hi, mid, lo;
      split3(x[c], hi, mid, lo);
      sB[0][0][c0 + c][m] = hi;
      sB[0][1][c0 + c][m] = mid;
      sB[0][2][c0 + c][m] = lo;
    }
  }

  const int nstep = d.nseg - 1;
  // pair j's slot: the hi / lo bf16 M (2 dk^2 elements, the 64 KiB of one
  // fp32 matrix) and S~
  auto m_at = [&](int j) { return Mseg + ((int64_t)(d.pair0 + j) * H + h) * (2 * mat); };
  auto st_at = [&](int j) { return Stseg + ((int64_t)(d.pair0 + j) * H + h) * mat; };
  // the inputs of step j (clamped to the last)
  auto load = [&](ScanInBf16 &in, int j) {
    j = min(j, nstep - 1);
    const bf16 *mj = m_at(j);
    // block ((w / 2) * 4 + s) * 2 + w % 2 of each part (scan_m_bf16_index)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int p = 0; p < 2; ++p)
        in.a[s][p] = *reinterpret_cast<const bf16x8 *>(
            mj + p * mat + ((((w >> 1) * 4 + s) * 2 + (w & 1)) * 64 + lane) * 8);
    const float *sr = st_at(j) + (16 * w + 4 * kq) * kD + col0 + n;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      in.st[e] = sr[e * kD];
  };
  // step j: reads sB[j & 1] and the inputs in `cur`, writes sB[(j + 1) & 1]
  // and Sin[sin0 + j + 1]; `ahead` takes the inputs of step j + kScanBf16Ahead
  auto step = [&](const ScanInBf16 &cur, ScanInBf16 &ahead, int j) {
    // B operands: rows 32 s + 8 kq .. + 7 of column n, each part
    Frag<bf16> b[4][3];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int p = 0; p < 3; ++p)
        b[s][p].v = *reinterpret_cast<const bf16x8 *>(&sB[j & 1][p][n][32 * s + 8 * kq]);
    load(ahead, j + kScanBf16Ahead);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      Frag<bf16> ah, al;
      ah.v = cur.a[s][0];
      al.v = cur.a[s][1];
      mma(acc, ah, b[s][0]);
      mma(acc, ah, b[s][1]);
      mma(acc, ah, b[s][2]);
      mma(acc, al, b[s][0]);
    }
    float *dst = sin + ((int64_t)(d.sin0 + j + 1) * H + h) * mat + col0 + n;
    const int r0 = 16 * w + 4 * kq;
    bf16x4 ph, pm, pl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += cur.st[e];
      bf16 hi, mid, lo;
      split3(acc[e], hi, mid, lo);
      ph[e] = hi;
      pm[e] = mid;
      pl[e] = lo;
      dst[(r0 + e) * kD] = acc[e];
    }
    *reinterpret_cast<bf16x4 *>(&sB[(j + 1) & 1][0][n][r0]) = ph;
    *reinterpret_cast<bf16x4 *>(&sB[(j + 1) & 1][1][n][r0]) = pm;
    *reinterpret_cast<bf16x4 *>(&sB[(j + 1) & 1][2][n][r0]) = pl;
    __syncthreads();
  };

  // a ring of three input sets: step j reads set j % 3 and fills set
  // (j + 2) % 3, the one step j - 1 read
  static_assert(kScanBf16Ahead == 2, "the ring below holds three input sets");
  ScanInBf16 in0, in1, in2;
  if (w < 8 && nstep > 0) { // (no pairs: only the entry state is written)
    load(in0, 0);
    load(in1, 1);
  }
  __syncthreads();
  if (w == 8) {
    // L2 warm-up, kScanBf16Warm steps ahead of use: this column block's
    // eighth of the M slot (one 128-byte line per lane) and its 16 columns
    // of S~ (64 bytes of each row), as loads into an LDS area nobody reads,
    // so that they sit in this wave's memory counter only.  One barrier per
    // step, as the compute waves; the loads are waited for before the wave
    // ends (they write this workgroup's LDS).
    const int cb = rem >> 3;
    auto warm = [&](int jw) {
      const __amdgpu_buffer_rsrc_t rm = buffer_rsrc(m_at(jw), (uint32_t)(4 * mat));
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(st_at(jw), (uint32_t)(4 * mat));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rm, (__attribute__((address_space(3))) void *)sWarm, 4, (cb * 64 + lane) * 128, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 2; ++r)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void *)sWarm, 4,
            ((64 * r + lane) * kD + col0) * 4, 0, 0, 0);
    };
    for (int jw = 2; jw < min(kScanBf16Warm, nstep); ++jw)
      warm(jw);
    for (int jj = 0; jj < nstep; ++jj) {
      if (jj + kScanBf16Warm < nstep)
        warm(jj + kScanBf16Warm);
      asm volatile("s_barrier" ::: "memory");
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return;
  }
  int j = 0;
  for (; j + 3 <= nstep; j += 3) {
    step(in0, in2, j);
    step(in1, in0, j + 1);
    step(in2, in1, j + 2);
  }
  if (j < nstep)
    step(in0, in2, j);
  if (j + 1 < nstep)
    step(in1, in0, j + 1);
}

// ---------------------------------------------------------------------------
// Output norm and gate as a pass of its own over o, in place ("Kimi K3.1 Pro
// 架构完全拆解" §3.3): o <- sigmoid(gate) w o / sqrt(mean(o^2) + eps) per
// (token, head) row.  For calls whose state chain runs 64-column blocks
// (few chains), where a whole row is no single workgroup's.  16 threads per
// row, 8 channels each (16-byte bf16 loads); HBM-bound.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void out_norm_gate_kernel(T *__restrict__ o,
                                                                 const T *__restrict__ gate,
                                                                 const float *__restrict__ w,
                                                                 float eps, int64_t rows) {
  const int part = threadIdx.x & 15;
  float wn[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    wn[j] = w ? w[8 * part + j] : 1.f;
  // the 16 threads of a row stay together (same r), so the row reduction
  // below only ever reads active lanes
  for (int64_t r = (int64_t)blockIdx.x * (kThreads / 16) + (threadIdx.x >> 4); r < rows;
       r += (int64_t)gridDim.x * (kThreads / 16)) {
    T *op = o + r * kD + 8 * part;
    float x[8], z[8];
    frag_to_f32(load_frag(op), x);
    frag_to_f32(load_frag(gate + r * kD + 8 * part), z);
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      ss += x[j] * x[j];
#pragma unroll
    for (int m = 1; m < 16; m <<= 1)
      ss += __shfl_xor(ss, m);
    const float sc = __builtin_amdgcn_rsqf(ss * (1.f / kD) + eps);
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      y[j] = x[j] * sc * wn[j] *
             __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z[j] * 1.4426950408889634f));
    store8(op, y);
  }
}

hipError_t launch_out_norm_gate(int elt, int64_t rows, void *o, const Epilogue &epi,
                                hipStream_t s) {
  if (rows == 0)
    return hipSuccess;
  const int64_t groups = (rows + kThreads / 16 - 1) / (kThreads / 16);
  const unsigned grid = (unsigned)std::min<int64_t>(groups, (int64_t)kComputeUnits * 8);
  if (elt == 1)
    out_norm_gate_kernel<bf16><<<grid, kThreads, 0, s>>>((bf16 *)o, (const bf16 *)epi.gate,
                                                          epi.weight, epi.eps, rows);
  else
    out_norm_gate_kernel<float><<<grid, kThreads, 0, s>>>((float *)o, (const float *)epi.gate,
                                                           epi.weight, epi.eps, rows);
  return hipGetLastError();
}

bool k2_fuses_epilogue(int32_t nchains, int32_t H) {
  return (int64_t)nchains * H * (kD / kBVWide) >= kComputeUnits;
}

hipError_t launch_k1(int elt, const ChunkDesc *chunks, int32_t nchunks, int32_t H,
                     const void *q, const void *k, const void *g, const void *beta, void *ws,
                     const Prologue &pro, hipStream_t s) {
  if (nchunks == 0)
    return hipSuccess;
  if (elt == 1)
    return launch_prep_bf16(chunks, nchunks, H, q, k, g, beta, ws, pro, s);
  // persistent grid: as many workgroups as are resident at once (LDS
  // limits fp32 to 1 per compute unit), each walking its items
  const int64_t nitems = (int64_t)nchunks * H;
  const int64_t resident = (int64_t)kComputeUnits;
  dim3 grid((unsigned)std::min(nitems, resident)), block(kThreads);
  // without q, k stands in as a readable buffer of the same shape
  const int has_q = q != nullptr;
  const void *qq = has_q ? q : k;
  auto launch = [&](auto kern) {
    kern<<<grid, block, 0, s>>>(chunks, H, (const float *)qq, (const float *)k,
                                (const float *)g, (const float *)beta, (uint8_t *)ws, has_q,
                                (int32_t)nitems, pro.A_log, pro.g_min, pro.qk_eps);
  };
  if (pro.on())
    launch(k1_kernel<float, true>);
  else
    launch(k1_kernel<float, false>);
  return hipGetLastError();
}

template <int BV, int NCT, int NB16, bool EPI>
static void launch_k2_bv(int elt, int mode, const ChainDesc *chains, int32_t nchains,
                         int32_t H, const uint8_t *w, const void *v, void *o,
                         const float *init, const float *sin, float *final_a, float *final_b,
                         int32_t mso, const Epilogue &epi, hipStream_t s) {
  // bf16 records: NB16 LDS record buffers; fp32 records: one (two do not fit)
  const int64_t npairs = (int64_t)nchains * H;
  const int64_t ncb = (mode == 1 ? 2 * kD : kD) / BV;
  dim3 grid((unsigned)((npairs + 7) / 8 * 8 * ncb)), block(k2_threads(BV, NCT));
  const int32_t np = (int32_t)npairs;
  // with the output epilogue, bf16 runs one tile per wave (8 waves) and fp32
  // two (4 waves: a wave per SIMD, whose registers its fp32 fragments need)
  constexpr bool kBf16 = !EPI || NCT == 1, kF32 = !EPI || NCT == 2;
  if (elt == 1) {
    if constexpr (kBf16) {
    if (mode == 1)
      k2_kernel<bf16, 1, BV, NCT, NB16, false><<<grid, block, 0, s>>>(
          chains, np, H, w, (const bf16 *)v, (bf16 *)o, init, sin, final_a, final_b, mso,
          nullptr, nullptr, 0.f);
    else
      k2_kernel<bf16, 0, BV, NCT, NB16, EPI><<<grid, block, 0, s>>>(
          chains, np, H, w, (const bf16 *)v, (bf16 *)o, init, sin, final_a, final_b, mso,
          (const bf16 *)epi.gate, epi.weight, epi.eps);
    }
  } else if constexpr (kF32) {
    if (mode == 1)
      k2_kernel<float, 1, BV, NCT, 1, false><<<grid, block, 0, s>>>(
          chains, np, H, w, (const float *)v, (float *)o, init, sin, final_a, final_b, mso,
          nullptr, nullptr, 0.f);
    else
      k2_kernel<float, 0, BV, NCT, 1, EPI><<<grid, block, 0, s>>>(
          chains, np, H, w, (const float *)v, (float *)o, init, sin, final_a, final_b, mso,
          (const float *)epi.gate, epi.weight, epi.eps);
  }
}

hipError_t launch_k2(int elt, int mode, const ChainDesc *chains, int32_t nchains, int32_t H,
                     const void *ws, const void *v, void *o, const float *init,
                     const float *sin, float *final_a, float *final_b, int m_scan_order,
                     const Epilogue &epi, hipStream_t s) {
  if (nchains == 0)
    return hipSuccess;
  const int32_t mso = mode == 1 ? m_scan_order : 0;
  const int64_t width = mode == 1 ? 2 * kD : kD;
  const int64_t wide_groups = (int64_t)nchains * H * (width / kBVWide);
  const uint8_t *w = (const uint8_t *)ws;
  if (mode == 0 && epi.on()) { // the output norm needs whole rows: the wide block
    if (elt == 1)
      launch_k2_bv<kBVWide, 1, 2, true>(elt, mode, chains, nchains, H, w, v, o, init, sin,
                                        final_a, final_b, mso, epi, s);
    else
      launch_k2_bv<kBVWide, 2, 1, true>(elt, mode, chains, nchains, H, w, v, o, init, sin,
                                        final_a, final_b, mso, epi, s);
  }
  else if (wide_groups < kComputeUnits)
    launch_k2_bv<kBVNarrow, 1, 2, false>(elt, mode, chains, nchains, H, w, v, o, init, sin,
                                         final_a, final_b, mso, epi, s);
  else if (mode == 0 || wide_groups < kK2ThroughputGroups)
    launch_k2_bv<kBVWide, 1, 2, false>(elt, mode, chains, nchains, H, w, v, o, init, sin,
                                       final_a, final_b, mso, epi, s);
  else // the segment pass of many segments: two single-buffered workgroups per CU
    launch_k2_bv<kK2ThroughputBV, kK2ThroughputNCT, 1, false>(
        elt, mode, chains, nchains, H, w, v, o, init, sin, final_a, final_b, mso, epi, s);
  return hipGetLastError();
}

hipError_t launch_scan(int elt, const ScanDesc *descs, int32_t ndesc, int32_t H,
                       const float *Mseg, const float *Stseg, const float *init, float *sin,
                       hipStream_t s) {
  if (ndesc == 0)
    return hipSuccess;
  const int64_t pairs = (int64_t)ndesc * H;
  const unsigned grid = (unsigned)((pairs + 7) / 8 * 8 * (kD / kScanBV));
  if (elt == 1)
    scan_bf16_kernel<<<grid, kScanBf16Threads, 0, s>>>(descs, ndesc, H, (const bf16 *)Mseg,
                                                        Stseg, init, sin);
  else
    scan_kernel<false><<<grid, kThreads, 0, s>>>(descs, ScanDesc{}, ndesc, H, Mseg, Stseg, init,
                                                 sin);
  return hipGetLastError();
}

hipError_t launch_scan_rows(int32_t nsteps, int32_t H, const float *M, const float *St,
                            const float *init, float *sin, hipStream_t s) {
  const ScanDesc one{0, nsteps + 1, 0, init ? 0 : -1};
  const unsigned grid = (unsigned)(((int64_t)H + 7) / 8 * 8 * (kD / kScanBV));
  scan_kernel<true><<<grid, kThreads, 0, s>>>(nullptr, one, 1, H, M, St, init, sin);
  return hipGetLastError();
}

} // namespace kda
