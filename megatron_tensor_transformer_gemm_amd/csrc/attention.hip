// Head-local scaled dot-product attention for gfx950 (the "attention core" of a
// tensor-parallel rank: its heads' softmax and value mixing need no communication,
// "7.9 Tensor and pipeline parallelism", section 2.2).
//
// O_j = softmax(Q_j K_j^T / sqrt(d_h) [+ causal mask]) V_j for each local query head j,
// grouped-query heads reading KV head j / (h_t / kv_t), each sequence on its own.
//
// One workgroup = 2 waves = 64 queries of one head of one sequence; each wave owns 32
// queries.  Keys are visited in blocks of 64 with a running (online) softmax:
//   S^T = K . Q^T         v_mfma_f32_32x32x16_bf16, keys on the rows, queries on the
//                          columns, so each lane holds one query's scores;
//   P^T = exp2(S^T - m)   row statistics need one exchange between lanes l and l^32;
//   O^T += V^T . P^T      P^T is already in the B-operand layout (the key order inside
//                          each 16-key step is the same permutation on both operands);
//                          V stays row-major in LDS and ds_read_b64_tr_b16 delivers
//                          V^T fragments.
// K and V blocks stream HBM/L2 -> LDS with buffer_load ... lds into two stages.  Keys
// beyond the sequence come back as zeros and are masked to -inf.
#include "tp_internal.h"

namespace tpk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_raw __attribute__((__vector_size__(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kBQ = 64;     // queries per workgroup (2 waves x 32)
constexpr int kBKV = 64;    // keys per block
constexpr uint32_t kOOB = 0x40000000u;
constexpr int kNumRecords = 0x40000000;
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, kNumRecords,
                                           kRsrcWord3);
}

// K tile [64 keys][DH]: chunk c of row r stored at c ^ (r & 15) (mod chunks per row).
template <int CPR>
__device__ __forceinline__ int swz_k(int r) { return r & (CPR - 1) & 15; }
// V tile [64 keys][DH], read by 4-row transposing reads: XOR pattern by row mod 4.
__device__ __forceinline__ int swz_v(int r) { return (0xCA60 >> (4 * (r & 3))) & 15; }

__device__ __forceinline__ float xor32(float v) {
  return __shfl_xor(v, 32, 64);
}

template <int DH>
__global__ void __launch_bounds__(128) attention_kernel(AttnDesc a) {
  constexpr int CPR = DH / 8;                 // 16-byte chunks per row
  constexpr int ROWB = DH * 2;                // bytes per row
  constexpr int TILE = kBKV * ROWB;           // bytes of one K or V tile
  constexpr int LD_PER_WAVE = TILE / 1024 / 2;
  constexpr int KS = DH / 16;                 // 16-wide k-steps over the head dimension
  constexpr int DB = DH / 32;                 // 32-row blocks of O^T
  static_assert(DH == 64 || DH == 128, "head_dim 64 or 128");

  __shared__ __attribute__((aligned(1024))) unsigned char kv0[2 * TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char kv1[2 * TILE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = a.seq_len;
  const int nqb = (S + kBQ - 1) / kBQ;
  const int qb = nqb - 1 - (int)blockIdx.x;   // heaviest (latest) query blocks first
  const int j = blockIdx.y;                   // local query head
  const int64_t seq = blockIdx.z;
  const int kvh = j / (a.h_t / a.kv_t);
  const int q0 = qb * kBQ;
  const int64_t row0 = seq * (int64_t)S;      // first token row of this sequence

  const __bf16* Qp = a.q + row0 * a.ldq + (int64_t)j * DH;
  const __bf16* Kp = a.k + row0 * a.ldkv + (int64_t)kvh * DH;
  const __bf16* Vp = a.v + row0 * a.ldkv + (int64_t)kvh * DH;

  // ---- Q fragments of this wave's 32 queries (B operand of S^T = K Q^T)
  const int qrow = q0 + wave * 32 + (lane & 31);
  bf16x8 qf[KS];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qp);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t off =
          qrow < S ? (uint32_t)((int64_t)qrow * a.ldq + 16 * ks + 8 * (lane >> 5)) * 2u : kOOB;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- K/V copy descriptors: copy q of a tile covers rows 1024/ROWB * q ..
  uint32_t ld_off[LD_PER_WAVE];
  int ld_row[LD_PER_WAVE];
#pragma unroll
  for (int i = 0; i < LD_PER_WAVE; ++i) {
    const int q = wave * LD_PER_WAVE + i;
    const int pos = q * 64 + lane;
    const int row = pos / CPR;
    const int c = (pos % CPR) ^ swz_k<CPR>(row);
    ld_off[i] = (uint32_t)(row * a.ldkv + 8 * c) * 2u;
    ld_row[i] = row;
  }
  // V copies use the V swizzle.
  uint32_t lv_off[LD_PER_WAVE];
#pragma unroll
  for (int i = 0; i < LD_PER_WAVE; ++i) {
    const int q = wave * LD_PER_WAVE + i;
    const int pos = q * 64 + lane;
    const int row = pos / CPR;
    const int c = (pos % CPR) ^ (swz_v(row) & (CPR - 1));
    lv_off[i] = (uint32_t)(row * a.ldkv + 8 * c) * 2u;
  }
  auto issue = [&](int kb, LDS_AS unsigned char* base) {
    const int key0 = kb * kBKV;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kp + (int64_t)key0 * a.ldkv);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vp + (int64_t)key0 * a.ldkv);
#pragma unroll
    for (int i = 0; i < LD_PER_WAVE; ++i) {
      const uint32_t v = key0 + ld_row[i] < S ? ld_off[i] : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (LDS_AS void*)(base + (wave * LD_PER_WAVE + i) * 1024), 16, v, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < LD_PER_WAVE; ++i) {
      const uint32_t v = key0 + ld_row[i] < S ? lv_off[i] : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (LDS_AS void*)(base + TILE + (wave * LD_PER_WAVE + i) * 1024), 16, v, 0, 0, 0);
    }
  };

  // ---- per-lane LDS read offsets
  // K (A operand of S^T): row = kblk*32 + lane%32, chunk 2*ks + lane/32
  const int krow = lane & 31;
  // V^T (A operand of O^T): 16-lane group g reads 4 key rows x 16 dh columns
  const int g4 = lane >> 4, i16 = lane & 15;
  const int vrow_l = 4 * (g4 >> 1) + (i16 >> 2);      // + 32*kblk + 16*h (+8 for the 2nd read)
  const int vsw = swz_v(vrow_l) & (CPR - 1);

  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) o[d] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float scale = 1.4426950408889634f / sqrtf((float)DH);   // log2(e) / sqrt(d_h)

  const int kend = a.causal ? (q0 + kBQ < S ? q0 + kBQ : S) : S;
  const int nkb = (kend + kBKV - 1) / kBKV;

  auto block = [&](int kb, const LDS_AS unsigned char* Ks) {
    const LDS_AS unsigned char* Vs = Ks + TILE;
    const int key0 = kb * kBKV;
    // S^T for 2 blocks of 32 keys
    f32x16 s[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      s[h] = f32x16{};
      const int r = h * 32 + krow;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = 2 * ks + (lane >> 5);
        const bf16x8 kf =
            *(const LDS_AS bf16x8*)(Ks + r * ROWB + ((c ^ swz_k<CPR>(r)) << 4));
        s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[h], 0, 0, 0);
      }
    }
    // mask, scale, running max (this lane's query: qrow)
    float mx = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 32 * h + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const bool masked = key >= S || (a.causal && key > qrow);
        const float v = masked ? -INFINITY : s[h][r] * scale;
        s[h][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float sum = 0.0f;
    bf16x8 pf[4];   // P^T fragments: 16-key steps (h, half)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = exp2f(s[h][8 * hf + e] - m_use);
          sum += p;
          pf[2 * h + hf][e] = (__bf16)p;
        }
    sum += xor32(sum);
    l_run = l_run * alpha + sum;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < DB; ++d) o[d] *= alpha;
    // O^T += V^T . P^T over 4 steps of 16 keys
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int h = st >> 1, hf = st & 1;
      const int rbase = 32 * h + 16 * hf + vrow_l;
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        const int n = d * 32 + 16 * (g4 & 1) + 4 * (i16 & 3);
        const int coff = (((n >> 3) ^ vsw) << 4) + ((n >> 2) & 1) * 8;
        const LDS_AS unsigned char* p0 = Vs + rbase * ROWB + coff;
        bf16x4_raw lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)p0);
        bf16x4_raw hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)(p0 + 8 * ROWB));
        const bf16x8 vf = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[st], o[d], 0, 0, 0);
      }
    }
  };

  LDS_AS unsigned char* S0 = (LDS_AS unsigned char*)kv0;
  LDS_AS unsigned char* S1 = (LDS_AS unsigned char*)kv1;
  issue(0, S0);
  int kb = 0;
  for (; kb + 1 < nkb; kb += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    issue(kb + 1, S1);
    block(kb, S0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kb + 2 < nkb) issue(kb + 2, S0);
    block(kb + 1, S1);
  }
  if (kb < nkb) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    block(kb, S0);
  }

  // ---- O = O^T / l, one 8-byte store per 4 consecutive head dims
  if (qrow < S) {
    const float inv = 1.0f / l_run;
    __bf16* Op = a.o + (row0 + qrow) * a.ldo + (int64_t)j * DH;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dh = d * 32 + 8 * g + 4 * (lane >> 5);
        *(bf16x4*)(Op + dh) = bf16x4{(__bf16)(o[d][4 * g] * inv), (__bf16)(o[d][4 * g + 1] * inv),
                                     (__bf16)(o[d][4 * g + 2] * inv), (__bf16)(o[d][4 * g + 3] * inv)};
      }
  }
}

}  // namespace

hipError_t launch_attention(const AttnDesc& a, hipStream_t s) {
  if (a.seq_len <= 0 || a.n_seq <= 0) return hipSuccess;
  if (a.n_seq > 65535 || a.h_t > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((a.seq_len + kBQ - 1) / kBQ), (unsigned)a.h_t, (unsigned)a.n_seq);
  if (a.head_dim == 128)
    hipLaunchKernelGGL(attention_kernel<128>, grid, dim3(128), 0, s, a);
  else if (a.head_dim == 64)
    hipLaunchKernelGGL(attention_kernel<64>, grid, dim3(128), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tpk
