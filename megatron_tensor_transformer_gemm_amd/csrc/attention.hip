// Head-local scaled dot-product attention for gfx950 (the "attention core" of a
// tensor-parallel rank: its heads' softmax and value mixing need no communication,
// "7.9 Tensor and pipeline parallelism", section 2.2).
//
// O_j = softmax(Q_j K_j^T / sqrt(d_h) [+ causal mask]) V_j for each local query head j,
// grouped-query heads reading KV head j / (h_t / kv_t), each sequence on its own.
//
// One workgroup = 8 waves = 64 queries of one head of one sequence.  A rank holds few
// heads, so there are few such query blocks; to keep the CUs busy the keys are split as
// well: the waves form 4 key groups of 2, group g visits the 32-key blocks g, g+4, g+8, ...
// and inside a group each wave owns 32 of the 64 queries.  Both waves of a group read the
// same K/V block from LDS, so every byte brought from L2 feeds 64 queries.
//   S^T = K . Q^T         v_mfma_f32_32x32x16_bf16, keys on the rows, queries on the
//                          columns, so each lane holds one query's scores;
//   P^T = exp2(S^T - m)   running (online) softmax in base 2 with the 1/sqrt(d_h) scale
//                          folded into one FMA; row statistics combine lanes l and l^32
//                          with v_permlane32_swap;
//   O^T += V^T . P^T      P^T is already in the B-operand layout (the key order inside
//                          each 16-key step is the same permutation on both operands);
//                          V stays row-major in LDS and ds_read_b64_tr_b16 delivers
//                          V^T fragments.
// The softmax is VALU work (a quarter-rate exp per score) of about the same length as the
// two products, so each wave runs it one block behind: while the MFMAs of block i's S^T
// run, the VALU turns block i-1's scores into P^T, then block i-1's O^T update follows.
// V therefore lags K by one block in the LDS stages.  The running maximum moves only when
// a block exceeds it by more than 2^8 (the exponentials stay below 256, the sums exact),
// so the O^T rescale is rare after the first blocks.
// K and V blocks stream L2 -> LDS with buffer_load ... lds, two stages each, issued by
// waves 0-3 only (each also brings the blocks of its partner on the same SIMD, wave + 4);
// keys beyond the sequence come back as zeros and are masked to -inf.  At the end the four groups'
// partial states (m, l, O^T) meet in LDS: wave (g, half) rescales and sums the four
// partials of head-dimension block g of its 32 queries and stores it.
//
// Ring step (context parallelism: "7.9 Tensor and pipeline parallelism" section 6,
// "Tensor & Pipeline Parallelism" (S17) "Sequence / ring attention"): the same kernel with
// a position offset between the query and key chunks (causal masking compares positions)
// and an epilogue that merges the chunk's normalised output and log-denominator into a
// running fp32 state instead of writing O.
#include "tp_internal.h"
#include "lds_copy.h"

namespace tpk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_raw __attribute__((__vector_size__(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kWaves = 8;
constexpr int kGroups = 4;     // key groups of 2 waves
constexpr int kBQ = 64;        // queries per workgroup
constexpr int kBK = 32;        // keys per block

// K block [32 keys][DH]: chunk c of row r stored at c ^ (r mod chunks-per-row, mod 16).
template <int CPR>
__device__ __forceinline__ int swz_k(int r) { return r & (CPR - 1) & 15; }
// V block [32 keys][DH], read by 4-row transposing reads: XOR pattern by row mod 4.
__device__ __forceinline__ int swz_v(int r) { return (0xCA60 >> (4 * (r & 3))) & 15; }

// Combine the values of lanes l and l^32 (the two halves of a score column).
__device__ __forceinline__ float max_pair(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_pair(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

constexpr float kLazy = 8.0f;  // log2 of the largest exponential kept before rescaling

// RING: fold the keys into the running state (o_state, lse_state) instead of writing O.
template <int DH, bool RING>
__global__ void __launch_bounds__(kWaves * 64) attention_kernel(AttnDesc a, int nqb, int strands) {
  constexpr int CPR = DH / 8;           // 16-byte chunks per row
  constexpr int ROWB = DH * 2;          // bytes per row
  constexpr int TILE = kBK * ROWB;      // one K or V block
  constexpr int NC = TILE / 1024 / 2;   // 1 KiB copies per wave per block
  constexpr int KS = DH / 16;           // 16-wide k-steps over the head dimension
  constexpr int DB = DH / 32;           // 32-row blocks of O^T
  constexpr int SLOT = 32 * 32 * 4;     // one fp32 32x32 block of O^T
  static_assert(DH == 64 || DH == 128, "head_dim 64 or 128");
  static_assert(2 * TILE == DB * SLOT, "two stages hold one half's partials");

  // K and V stages: [stage][group][block].  After the key loop kst holds the partial
  // O^T blocks of the first 32 queries, vst those of the second.
  __shared__ __attribute__((aligned(1024))) unsigned char kst[2 * kGroups * TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vst[2 * kGroups * TILE];
  __shared__ f32x2 ml[2 * kGroups * 64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = wave >> 1;    // key group
  const int qh = wave & 1;    // which 32 of the 64 queries
  const int S = a.seq_len;
  // Workgroups are dealt round-robin over the 8 XCDs.  With `strands` = G > 0 each head's
  // query blocks form G strands (qb mod G), heaviest first, h_t*G a multiple of 8: XCD x
  // takes h_t*G/8 adjacent strands (the K/V of at most two heads through its L2), and its
  // slot i runs level i / (strands per XCD), so every XCD proceeds heaviest first.
  // Otherwise (G = 0): latest (heaviest) block positions first, all heads of a position
  // together.
  int j, qb;
  if (strands > 0) {
    const int spx = a.h_t * strands / 8;
    const int x = (int)(blockIdx.x & 7u), i = (int)(blockIdx.x >> 3);
    const int sidx = x * spx + i % spx;
    j = sidx / strands;
    qb = nqb - strands + sidx % strands - strands * (i / spx);
  } else {
    qb = nqb - 1 - (int)(blockIdx.x / (unsigned)a.h_t);
    j = (int)(blockIdx.x % (unsigned)a.h_t);
  }
  const int64_t seq = blockIdx.y;
  const int kvh = j / (a.h_t / a.kv_t);
  const int q0 = qb * kBQ;
  const int64_t row0 = seq * (int64_t)S;   // first token row of this sequence

  const __bf16* Qp = a.q + row0 * a.ldq + (int64_t)j * DH;
  const __bf16* Kp = a.k + row0 * a.ldkv + (int64_t)kvh * DH;
  const __bf16* Vp = a.v + row0 * a.ldkv + (int64_t)kvh * DH;

  // ---- Q fragments of this wave's 32 queries (B operand of S^T = K Q^T)
  const int qrow = q0 + 32 * qh + (lane & 31);
  // Ring step: this row's log-denominator so far, read before any wave can overwrite it
  float lse_old = -INFINITY;
  if (RING && qrow < S) lse_old = a.lse_state[(row0 + qrow) * a.ld_lse + j];
  bf16x8 qf[KS];
  {
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16*>(Qp), (short)0, kNumRecords, kRsrcWord3);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t off =
          qrow < S ? (uint32_t)((int64_t)qrow * a.ldq + 16 * ks + 8 * (lane >> 5)) * 2u : kOOB;
      qf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
    }
    // Retire these loads here: a wait for them inside the key loop would also wait for the
    // copies of the next block, which are in flight there.
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qf[ks]));
  }

  LDS_AS unsigned char* KST = (LDS_AS unsigned char*)kst;
  LDS_AS unsigned char* VST = (LDS_AS unsigned char*)vst;

  // ---- copies: each half of a group's K and V blocks is brought by the wave of that half
  // (qh) in groups 0 and 1, which also brings the same half for group g + 2 (the waves
  // w + 4, on the same SIMD as wave w since waves go to the SIMDs round-robin).  A wave
  // held at copy issue also slows the other wave of its SIMD; here that other wave has no
  // copies of its own to be held on (causal core at 2,048 tokens, 6 heads: 24.6 -> 22.6 us,
  // three alternations on one GPU).  Copy i covers rows c_row0 + i*RPC.  The V swizzle depends on the row mod
  // 4 only, so its offsets step by a constant; the K swizzle needs one offset per copy.
  constexpr int RPC = 64 / CPR;          // rows per 1 KiB copy
  const int c_row0 = (qh * NC * 64 + lane) / CPR, c_slot = lane % CPR;
  uint32_t k_off[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int row = c_row0 + i * RPC;
    k_off[i] = (uint32_t)(row * a.ldkv + 8 * (c_slot ^ swz_k<CPR>(row))) * 2u;
  }
  const uint32_t v_off0 = (uint32_t)(c_row0 * a.ldkv + 8 * (c_slot ^ (swz_v(c_row0) & (CPR - 1)))) * 2u;
  const uint32_t copy_step = (uint32_t)(RPC * a.ldkv) * 2u;
  static_assert(RPC % 4 == 0, "V swizzle period");
  // keys this block needs: causal stops after the last query's position
  const int kend = a.causal ? (q0 + kBQ + a.delta < S ? q0 + kBQ + a.delta : S) : S;
  if (RING && kend <= 0) return;   // every key lies after every query: the state stands
  const int nkb = (kend + kBK - 1) / kBK;
  const int nit = (nkb + kGroups - 1) / kGroups;   // same for every wave

  // This wave's half of block gg + 4*it of group gg (its K or its V) into stage it % 2.
  // Past the last block every lane is masked (zeros), so the product code runs
  // unconditionally on well-defined data.
  auto issue_group = [&](int gg, int it, bool is_v) {
    const int key0 = (gg + kGroups * it) * kBK;
    const int lim = key0 < kend ? S - key0 : 0;
    const i32x4 desc = make_desc((is_v ? Vp : Kp) + (int64_t)key0 * a.ldkv);
    const uint32_t base =
        (uint32_t)(uintptr_t)((is_v ? VST : KST) + ((it & 1) * kGroups + gg) * TILE);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const uint32_t off = is_v ? v_off0 + i * copy_step : k_off[i];
      copy16_to_lds(desc, c_row0 < lim - i * RPC ? off : kOOB,
                    __builtin_amdgcn_readfirstlane(base + (qh * NC + i) * 1024));
    }
  };
  static_assert(kWaves == 8 && kGroups == 4, "copying waves 0-3 cover groups g and g + 2");
  auto issue = [&](int it, bool is_v) {
    if (wave < 4) {
      issue_group(g, it, is_v);
      issue_group(g + 2, it, is_v);
    }
  };
  auto stage = [&](LDS_AS unsigned char* stages, int it) -> const LDS_AS unsigned char* {
    return stages + ((it & 1) * kGroups + g) * TILE;
  };

  // ---- per-lane LDS read offsets.  The XOR swizzles touch address bits inside a row
  // only, so the offset of k-step ks (of head-dim block d) is the base XOR a constant.
  // K (A operand of S^T): row = lane % 32, chunk 2*ks + lane / 32
  const int krow = lane & 31;
  const uint32_t k_rd = (uint32_t)(krow * ROWB + (((lane >> 5) ^ swz_k<CPR>(krow)) << 4));
  // V^T (A operand of O^T): 16-lane group g4 reads 4 key rows x 16 head-dim columns; the
  // second read of a fragment is 8 rows further.
  const int g4 = lane >> 4, i16 = lane & 15;
  const int vrow_l = 4 * (g4 >> 1) + (i16 >> 2);
  const int vsw = swz_v(vrow_l) & (CPR - 1);
  const int vn = 16 * (g4 & 1) + 4 * (i16 & 3);
  const uint32_t v_rd = (uint32_t)(vrow_l * ROWB + (((vn >> 3) ^ vsw) << 4) + ((vn >> 2) & 1) * 8);
  static_assert(ROWB >= 128 && (ROWB & (ROWB - 1)) == 0, "row pitch");

  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) o[d] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;   // running max (scaled, log2 units) and sum
  const float scale = 1.4426950408889634f / sqrtf((float)DH);   // log2(e) / sqrt(d_h)
  const int qmin = q0 + 32 * qh;                                 // this wave's first query

  // Does block `it` of this group reach past the sequence or the diagonal?
  auto needs_mask = [&](int it) {
    const int key0 = (g + kGroups * it) * kBK;
    return key0 + kBK > S || (a.causal && key0 + kBK - 1 > qmin + a.delta);
  };
  auto read_k = [&](const LDS_AS unsigned char* Ks, bf16x8 (&kf)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = *(const LDS_AS bf16x8*)(Ks + (k_rd ^ (ks << 5)));
  };
  auto read_v = [&](const LDS_AS unsigned char* Vs, bf16x8 (&vf)[2][DB]) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        const LDS_AS unsigned char* p0 = Vs + 16 * hf * ROWB + (v_rd ^ (d << 6));
        bf16x4_raw lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)p0);
        bf16x4_raw hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)(p0 + 8 * ROWB));
        vf[hf][d] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
  };
  auto qk = [&](const bf16x8 (&kf)[KS]) {
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s, 0, 0, 0);
    return s;
  };
  auto pv = [&](const bf16x8 (&vf)[2][DB], const bf16x8 (&pf)[2]) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int d = 0; d < DB; ++d)
        o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[hf][d], pf[hf], o[d], 0, 0, 0);
  };
  // Scores of block `it` (raw S^T) -> P^T fragments; updates m_run and l_run.  Returns
  // whether O^T must be rescaled by `alpha` (the same answer on every lane).
  auto softmax = [&](auto mask_t, f32x16 s, int it, bf16x8 (&pf)[2], float& alpha) {
    if constexpr (decltype(mask_t)::value) {
      const int key0 = (g + kGroups * it) * kBK;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (key >= S || (a.causal && key > qrow + a.delta)) s[r] = -INFINITY;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = max_pair(mx) * scale;
    const bool grow = __builtin_amdgcn_ballot_w64(mx > m_run + kLazy) != 0;
    const float m_new = grow ? fmaxf(m_run, mx) : m_run;
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float sum = 0.0f;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * hf + e], scale, -m_use));
        sum += p;
        pf[hf][e] = (__bf16)p;
      }
    l_run = __builtin_fmaf(l_run, alpha, sum_pair(sum));
    return grow;
  };
  auto rescale = [&](float alpha) {
#pragma unroll
    for (int d = 0; d < DB; ++d) o[d] *= alpha;
  };

  // ---- key loop: iteration it multiplies S^T of block it and finishes block it-1
  issue(0, false);
  sync_copies<0>();
  if (nit > 1) issue(1, false);
  issue(0, true);
  f32x16 s_a, s_b;
  {
    bf16x8 kf[KS];
    read_k(stage(KST, 0), kf);
    s_a = qk(kf);
  }
  // One iteration: scores s_in of block it-1 -> P^T and the O^T update, while the MFMAs
  // produce s_out, the scores of block it.
  auto step = [&](auto mask_t, int it, const f32x16& s_in, f32x16& s_out) {
    // K of block it and V of block it-1 have landed; every wave is done with the
    // previous iteration's stages
    sync_copies<0>();
    if (it + 1 < nit) issue(it + 1, false);
    issue(it, true);
    bf16x8 pf[2];
    float alpha;
    bool grow;
    {
      bf16x8 kf[KS];
      read_k(stage(KST, it), kf);
      s_out = qk(kf);
      grow = softmax(mask_t, s_in, it - 1, pf, alpha);
    }
    // V fragments only now: they take the K fragments' registers
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 vf[2][DB];
    read_v(stage(VST, it - 1), vf);
    if (grow) rescale(alpha);
    pv(vf, pf);
  };
  // Blocks that need a mask (past the diagonal or the sequence end) come last; the loop
  // over the others is unrolled by two so the score registers alternate without copies.
  int it = 1;
  int it_nm = 1;   // first iteration whose finished block needs a mask
  while (it_nm < nit && !needs_mask(it_nm - 1)) ++it_nm;
  for (; it + 1 < it_nm; it += 2) {
    step(Flag<false>{}, it, s_a, s_b);
    step(Flag<false>{}, it + 1, s_b, s_a);
  }
  if (it < it_nm) {
    step(Flag<false>{}, it, s_a, s_b);
    s_a = s_b;
    ++it;
  }
  for (; it < nit; ++it) {
    step(Flag<true>{}, it, s_a, s_b);
    s_a = s_b;
  }
  sync_copies<0>();
  {
    bf16x8 vf[2][DB], pf[2];
    read_v(stage(VST, nit - 1), vf);
    float alpha;
    const bool grow = needs_mask(nit - 1) ? softmax(Flag<true>{}, s_a, nit - 1, pf, alpha)
                                          : softmax(Flag<false>{}, s_a, nit - 1, pf, alpha);
    if (grow) rescale(alpha);
    pv(vf, pf);
  }

  // ---- combine the four groups' partial states
  sync_copies<0>();
  LDS_AS unsigned char* half = qh ? VST : KST;
  ((LDS_AS f32x2*)ml)[(qh * kGroups + g) * 64 + lane] = f32x2{m_run, l_run};
#pragma unroll
  for (int d = 0; d < DB; ++d)
    if (d != g) {
      LDS_AS f32x4* p = (LDS_AS f32x4*)(half + (g * DB + d) * SLOT);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        p[r4 * 64 + lane] = f32x4{o[d][4 * r4], o[d][4 * r4 + 1], o[d][4 * r4 + 2], o[d][4 * r4 + 3]};
    }
  sync_copies<0>();
  if (g >= DB) return;   // head_dim 64: groups 2 and 3 only contribute

  float mg[kGroups], lg[kGroups];
#pragma unroll
  for (int h = 0; h < kGroups; ++h) {
    const f32x2 t = ((const LDS_AS f32x2*)ml)[(qh * kGroups + h) * 64 + lane];
    mg[h] = t[0];
    lg[h] = t[1];
  }
  float M = mg[0];
#pragma unroll
  for (int h = 1; h < kGroups; ++h) M = fmaxf(M, mg[h]);
  const float Mu = M == -INFINITY ? 0.0f : M;
  float al[kGroups], L = 0.0f;
#pragma unroll
  for (int h = 0; h < kGroups; ++h) {
    al[h] = __builtin_amdgcn_exp2f(mg[h] - Mu);
    L += al[h] * lg[h];
  }
  const float inv = 1.0f / L;
#pragma unroll
  for (int d = 0; d < DB; ++d)
    if (d == g) {
      const float own = __builtin_amdgcn_exp2f(m_run - Mu);
      f32x16 acc = o[d] * own;
#pragma unroll
      for (int h = 0; h < kGroups; ++h)
        if (h != g) {
          const LDS_AS f32x4* p = (const LDS_AS f32x4*)(half + (h * DB + d) * SLOT);
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 t = p[r4 * 64 + lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[4 * r4 + i] += al[h] * t[i];
          }
        }
      if constexpr (RING) {
        // Merge (O_c = acc / L, lse_c = ln L + Mu ln 2) into the state: with
        // M = max(lse_old, lse_c) the weights are e^(lse - M), the new state the weighted
        // mean of the two outputs and M + ln(sum of weights).  A row with no visible key
        // in this chunk (L = 0) keeps its state.
        if (qrow < S && L > 0.0f) {
          constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
          const float lc = Mu + __builtin_amdgcn_logf(L);   // log2 units
          const float lo = lse_old * kLog2e;
          const float M2 = fmaxf(lo, lc);
          const float w_o = __builtin_amdgcn_exp2f(lo - M2), w_c = __builtin_amdgcn_exp2f(lc - M2);
          const float den = w_o + w_c;
          const float r_o = w_o / den, r_c = w_c * inv / den;
          float* St = a.o_state + (row0 + qrow) * a.ld_state + (int64_t)j * DH + 32 * d;
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            f32x4* sp = (f32x4*)(St + 8 * r4 + 4 * (lane >> 5));
            const f32x4 prev = *sp;
            *sp = f32x4{r_o * prev[0] + r_c * acc[4 * r4], r_o * prev[1] + r_c * acc[4 * r4 + 1],
                        r_o * prev[2] + r_c * acc[4 * r4 + 2], r_o * prev[3] + r_c * acc[4 * r4 + 3]};
          }
          if (g == 0) a.lse_state[(row0 + qrow) * a.ld_lse + j] = (M2 + __builtin_amdgcn_logf(den)) * kLn2;
        }
      } else if (qrow < S) {
        // O = O^T / l, one 8-byte store per 4 consecutive head dims
        __bf16* Op = a.o + (row0 + qrow) * a.ldo + (int64_t)j * DH + 32 * d;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *(bf16x4*)(Op + 8 * r4 + 4 * (lane >> 5)) =
              bf16x4{(__bf16)(acc[4 * r4] * inv), (__bf16)(acc[4 * r4 + 1] * inv),
                     (__bf16)(acc[4 * r4 + 2] * inv), (__bf16)(acc[4 * r4 + 3] * inv)};
      }
    }
}

}  // namespace

hipError_t launch_attention(const AttnDesc& a, hipStream_t s) {
  if (a.seq_len <= 0 || a.n_seq <= 0) return hipSuccess;
  const int64_t nqb = (a.seq_len + kBQ - 1) / kBQ;
  if (a.n_seq > 65535 || a.h_t <= 0 || nqb * a.h_t > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(nqb * a.h_t), (unsigned)a.n_seq);
  int g8 = 8;
  while (a.h_t % g8) g8 >>= 1;   // gcd(h_t, 8)
  const int strands = nqb % (8 / g8) == 0 ? 8 / g8 : 0;
  const bool ring = a.o == nullptr;
  if (ring && (a.o_state == nullptr || a.lse_state == nullptr)) return hipErrorInvalidValue;
  if (a.head_dim == 128 && !ring)
    hipLaunchKernelGGL((attention_kernel<128, false>), grid, dim3(kWaves * 64), 0, s, a, (int)nqb, strands);
  else if (a.head_dim == 64 && !ring)
    hipLaunchKernelGGL((attention_kernel<64, false>), grid, dim3(kWaves * 64), 0, s, a, (int)nqb, strands);
  else if (a.head_dim == 128)
    hipLaunchKernelGGL((attention_kernel<128, true>), grid, dim3(kWaves * 64), 0, s, a, (int)nqb, strands);
  else if (a.head_dim == 64)
    hipLaunchKernelGGL((attention_kernel<64, true>), grid, dim3(kWaves * 64), 0, s, a, (int)nqb, strands);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

namespace {

// Ring state set-up: one thread per 4 columns of a row (cols a multiple of 4), and the
// first `heads` threads of a row also clear its log-denominators.
__global__ void ring_init_kernel(float* o_state, float* lse_state, int64_t rows, int32_t cols,
                                 int32_t heads, int32_t ld_state, int32_t ld_lse) {
  const int64_t row = blockIdx.y + (int64_t)gridDim.y * blockIdx.z;
  if (row >= rows) return;
  const int c = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (4 * c < cols) *(f32x4*)(o_state + row * ld_state + 4 * c) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (c < heads) lse_state[row * ld_lse + c] = -INFINITY;
}

// O = bf16(state), round to nearest even, 4 columns per thread
__global__ void ring_finish_kernel(const float* o_state, __bf16* o, int64_t rows, int32_t cols,
                                   int32_t ld_state, int32_t ldo) {
  const int64_t row = blockIdx.y + (int64_t)gridDim.y * blockIdx.z;
  const int c = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (row >= rows || 4 * c >= cols) return;
  const f32x4 v = *(const f32x4*)(o_state + row * ld_state + 4 * c);
  *(bf16x4*)(o + row * ldo + 4 * c) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
}

// rows -> (y, z) grid dimensions within the 65535 limit of each
bool row_grid(int64_t rows, int32_t cols, dim3& grid) {
  const int64_t bx = (cols / 4 + 255) / 256;
  const int64_t gy = rows < 65535 ? rows : 65535;
  const int64_t gz = (rows + gy - 1) / gy;
  if (bx > 0x7FFFFFFF || gz > 65535) return false;
  grid = dim3((unsigned)(bx > 0 ? bx : 1), (unsigned)gy, (unsigned)gz);
  return true;
}

}  // namespace

hipError_t launch_ring_init(float* o_state, float* lse_state, int64_t rows, int32_t cols,
                            int32_t heads, int32_t ld_state, int32_t ld_lse, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  dim3 grid;
  if (cols % 4 || 4 * heads > cols || !row_grid(rows, cols, grid)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ring_init_kernel, grid, dim3(256), 0, s, o_state, lse_state, rows, cols, heads,
                     ld_state, ld_lse);
  return hipGetLastError();
}

hipError_t launch_ring_finish(const float* o_state, __bf16* o, int64_t rows, int32_t cols,
                              int32_t ld_state, int32_t ldo, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  dim3 grid;
  if (cols % 4 || !row_grid(rows, cols, grid)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ring_finish_kernel, grid, dim3(256), 0, s, o_state, o, rows, cols, ld_state, ldo);
  return hipGetLastError();
}

}  // namespace tpk
