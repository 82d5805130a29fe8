// Fused exact-attention forward for AMD CDNA4 (gfx950, MI355X), and its C ABI.
//
// What it computes: O = softmax(scale * Q K^T) V row-wise, plus the per-row
// natural-log LSE, for bf16 Q/K/V with fp32 accumulation ("FlashAttention-4"
// (papercache summary), section 2.1; "059 · FlashAttention" (wq-win),
// section 2).  The score tile S and probability tile P exist only in
// registers: each workgroup owns one block of query rows of one head and walks
// the key/value blocks with the online-softmax statistics of FlashAttention
// V1 到 V4 (chengxuchu), section 3.4.1 -- running max m, running sum l, and an
// unnormalised accumulator rescaled by exp(m_old - m_new), divided by l once at
// the end.  The work split (one workgroup per query block, inner loop over key
// blocks) is the FlashAttention-2 partitioning (chengxuchu, section 4.3).
//
// CDNA4 mapping
// -------------
// * 4 waves (wave64) per workgroup; each wave owns 32 query rows, so a
//   workgroup covers kBr = 128 query rows.
// * Scores are computed transposed, S^T = K Q^T, with
//   v_mfma_f32_32x32x16_bf16: A = a 32-key slice of K read from LDS, B = the
//   wave's 32 query rows held in VGPRs for the whole kernel.  In the 32x32
//   accumulator layout lane l holds column l%32 (one query row) and 16 of the
//   32 key rows; lanes l and l^32 hold the other half of the same row.  Row
//   max and row sum are therefore in-lane reductions plus one exchange with
//   lane l^32, and the row statistics are per-lane scalars.
// * The output is accumulated transposed too, O^T += V^T P^T, with the same
//   instruction: A = a 32(d) x 16(key) slice of V^T, B = P^T taken straight
//   from the score accumulators after conversion to bf16, so P never leaves
//   registers.  The 16 keys an instruction consumes must sit in the same
//   (lane-half, slot) positions in both operands; the score layout gives
//   lane-half g the keys {4g..4g+3, 8+4g..8+4g+3} of each 16-key group.  V
//   stays row-major in LDS and each A operand is assembled from two gfx950
//   transpose reads (ds_read_b64_tr_b16): in every 16-lane block, lane j
//   addresses 4 consecutive d of key row j/4 and lane i receives the 4 keys of
//   column i, which is exactly "4 consecutive keys of one d" per lane.
// * K and V tiles (row-major, padded rows) are double-buffered in LDS; the
//   next tile's global loads are issued into registers before the current
//   tile's MFMAs and written to the other buffer after them, so each key step
//   needs a single barrier.  Rows past the last needed key are loaded from a
//   clamped (valid) row and masked, so the loads need no predication.
// * Conditional rescaling (FlashAttention-4 (papercache summary), section
//   3.1.4): the running max of a row is raised, and O and l rescaled, only
//   when the new block's max exceeds it by more than tau = 8 (log2 units, a
//   factor of 256); otherwise the block is accumulated against the stale max
//   (probabilities up to 2^8 before normalisation).  The decision is made per
//   wavefront -- if any lane needs it, the whole wave rescales -- so the skip
//   is a uniform branch.  The final O / l and LSE = m + log2 l stay exact.
// * Softmax runs in the exp2 domain with scale*log2(e) folded into one FMA per
//   score; LSE is converted back to natural log in the epilogue.
// * Causal: key blocks past the query block's last row are never visited, and
//   a wave skips a key block lying wholly above its rows; masks are applied
//   only on blocks that cross the diagonal or the key tail.
// * Grid order: workgroup ids are assigned round-robin to the 8 XCDs, so the
//   id is first remapped to make each XCD's share a contiguous run of logical
//   work items; logical order is batch, KV head, query block (longest first
//   under the causal mask), then the query heads sharing that KV head, so the
//   workgroups resident on one XCD read the same K/V from its L2
//   (longest-processing-time-first scheduling and head grouping of
//   FlashAttention-4 (papercache summary), section 3.3).

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "attn.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBr = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kXcds = 8;                    // MI355X: 8 XCDs, 32 CUs each
constexpr float kLn2 = 0.693147180559945309f;

template <int D>
struct Tile {
  static constexpr int BC = (D == 64) ? 128 : 64;  // keys per step
  static constexpr int KT = BC / 32;               // 32-key MFMA blocks per step
  static constexpr int DT = D / 32;                // 32-wide d blocks of O^T
  static constexpr int KS = D / 16;                // 16-deep d slices of S^T
  static constexpr int KSTR = D + 8;               // LDS row stride of K (elements)
  static constexpr int VSTR = D + 16;              // LDS row stride of V (elements)
  static constexpr int K_ELEMS = BC * KSTR;
  static constexpr int V_ELEMS = BC * VSTR;
  static constexpr int BUF = K_ELEMS + V_ELEMS;  // one K + V buffer
  static constexpr int CHUNKS = BC * D / 8 / kThreads;  // 16-byte chunks per thread per tile
  static_assert(CHUNKS * kThreads * 8 == BC * D, "tile split");
};

constexpr float kTau = 8.0f;  // conditional-rescale threshold, log2 units
constexpr int kBufferFlags = 0x00020000;  // buffer resource word 3 for raw 32-bit access (gfx9)

struct Params {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  const int32_t* seqlens_k;  // padded form, may be null
  const int32_t* cu_q;       // packed form
  const int32_t* cu_k;
  int Hq, Hkv, G;
  int Nq, Nk;  // packed form: max_seqlen_q, max_seqlen_k
  int nqb;     // query blocks per (sequence, head)
  int num_seqs;
  float c;  // scale * log2(e)
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max(a, b, c) in one instruction.  fmaxf would make the compiler quiet
// possible signalling NaNs of the MFMA results first (an extra instruction per
// operand); scores here are finite or -inf.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Two transpose reads of LDS, concatenated into one 8-element bf16 operand.
__device__ __forceinline__ bf16x8 read_tr_pair(const __bf16* p0, const __bf16* p1) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(Params p) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * T::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  // ---- work item: XCD-contiguous remap, then (seq, kv head, q block, head in group)
  const int n = gridDim.x;
  const int bid = blockIdx.x;
  const int xcd = bid % kXcds;
  const int per = n / kXcds;
  const int rem = n % kXcds;
  int t = xcd * per + min(xcd, rem) + bid / kXcds;
  const int gi = t % p.G;
  t /= p.G;
  const int qbi = t % p.nqb;
  t /= p.nqb;
  const int hkv = t % p.Hkv;
  const int b = t / p.Hkv;
  const int qb = CAUSAL ? (p.nqb - 1 - qbi) : qbi;
  const int h = hkv * p.G + gi;

  int q_len, nk;
  long q_row0, k_row0, lse_base, lse_hstride;
  if (VARLEN) {
    const int qs = p.cu_q[b], qe = p.cu_q[b + 1];
    const int ks = p.cu_k[b], ke = p.cu_k[b + 1];
    q_len = min(max(qe - qs, 0), p.Nq);
    nk = min(max(ke - ks, 0), p.Nk);
    q_row0 = qs;
    k_row0 = ks;
    lse_base = qs;
    lse_hstride = p.cu_q[p.num_seqs];
  } else {
    q_len = p.Nq;
    nk = p.Nk;
    if (p.seqlens_k != nullptr) nk = min(max(p.seqlens_k[b], 0), p.Nk);
    q_row0 = (long)b * p.Nq;
    k_row0 = (long)b * p.Nk;
    lse_base = (long)b * p.Hq * p.Nq;
    lse_hstride = p.Nq;
  }
  const int q0 = qb * kBr;
  if (q0 >= q_len) return;  // uniform over the workgroup, before any barrier

  const long q_stride = (long)p.Hq * D;
  const long kv_stride = (long)p.Hkv * D;
  const __bf16* qbase = p.q + q_row0 * q_stride + (long)h * D;
  const __bf16* kbase = p.k + k_row0 * kv_stride + (long)hkv * D;
  const __bf16* vbase = p.v + k_row0 * kv_stride + (long)hkv * D;

  // ---- this lane's query row, held as the B operand of S^T = K Q^T
  const int qrow = q0 + wave * kRowsPerWave + l32;
  bf16x8 qf[T::KS];
  if (qrow < q_len) {
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qbase + qrow * q_stride + ks * 16 + 8 * g);
  } else {
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) qf[ks] = bf16x8{};
  }

  // Keys this workgroup needs: all visible keys of its rows.
  int kv_end = nk;
  if (CAUSAL) kv_end = min(nk, min(q0 + kBr, q_len));
  const int n_tiles = (kv_end + T::BC - 1) / T::BC;

  // ---- tile staging: global -> registers -> LDS (K and V alike, 16-byte chunks)
  // Buffer loads through a per-tile resource whose range ends at row kv_end:
  // rows past it read as zero (and are masked below), so the loads need no
  // predication and no per-lane 64-bit address arithmetic.
  const uint32_t row_bytes = static_cast<uint32_t>(kv_stride) * 2u;
  u32x4 kr[T::CHUNKS];
  u32x4 vr[T::CHUNKS];
  auto load_tile = [&](int kv0) {
    const int nrows = min(kv_end - kv0, T::BC);
    const int nbytes = nrows * static_cast<int>(row_bytes);
    const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16*>(kbase + kv0 * kv_stride), (short)0, nbytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16*>(vbase + kv0 * kv_stride), (short)0, nbytes, kBufferFlags);
#pragma unroll
    for (int c = 0; c < T::CHUNKS; ++c) {
      const int idx = tid + c * kThreads;
      const uint32_t off = (idx / (D / 8)) * row_bytes + (idx % (D / 8)) * 16u;
      kr[c] = __builtin_amdgcn_raw_buffer_load_b128(kres, off, 0, 0);
      vr[c] = __builtin_amdgcn_raw_buffer_load_b128(vres, off, 0, 0);
    }
  };
  auto store_tile = [&](__bf16* buf) {
#pragma unroll
    for (int c = 0; c < T::CHUNKS; ++c) {
      const int idx = tid + c * kThreads;
      const int row = idx / (D / 8);
      const int col = (idx % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(buf + row * T::KSTR + col) = kr[c];
      *reinterpret_cast<u32x4*>(buf + T::K_ELEMS + row * T::VSTR + col) = vr[c];
    }
  };

  // Per-lane offset of the V transpose reads: key row 4g + (l%16)/4 of each
  // 16-key group, d columns 16*((l/16)%2) + 4*(l%4) of each 32-wide d block.
  const int v_lane = (4 * g + (l32 & 15) / 4) * T::VSTR + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  f32x16 acc[T::DT];
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt) acc[dt] = f32x16{};
  float m_run = -INFINITY;  // running max, log2 domain (scores times scale*log2 e)
  float l_run = 0.f;        // this lane's half of the running sum
  const float c = p.c;
  const int wrow0 = q0 + wave * kRowsPerWave;
  const int wrow_last = wrow0 + kRowsPerWave - 1;

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(smem);
  }
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int kv0 = j * T::BC;
    const __bf16* cur = smem + (j & 1) * T::BUF;
    __bf16* nxt = smem + ((j + 1) & 1) * T::BUF;
    const bool has_next = j + 1 < n_tiles;
    if (has_next) load_tile(kv0 + T::BC);

    if (!CAUSAL || kv0 <= wrow_last) {  // uniform over the wave
      // S^T block kt: keys kv0+32kt.., queries of this wave.
      f32x16 s[T::KT];
#pragma unroll
      for (int kt = 0; kt < T::KT; ++kt) {
        s[kt] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(cur + (kt * 32 + l32) * T::KSTR +
                                                             ks * 16 + 8 * g);
          s[kt] = mfma32(a, qf[ks], s[kt]);
        }
      }
      // Masks, only on blocks crossing the key tail or the diagonal.
      const bool need_mask = (kv0 + T::BC > nk) || (CAUSAL && kv0 + T::BC - 1 > wrow0);
      if (need_mask) {
#pragma unroll
        for (int kt = 0; kt < T::KT; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + kt * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            const bool vis = key < nk && (!CAUSAL || key <= qrow);
            if (!vis) s[kt][r] = -INFINITY;
          }
      }
      // Row max: in-lane (two independent chains), then with the partner lane.
      float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < T::KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          mx0 = max3f(mx0, s[kt][r], s[kt][r + 1]);
          mx1 = max3f(mx1, s[kt][r + 2], s[kt][r + 3]);
        }
      float mx = max3f(mx0, mx1, -INFINITY);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * c;
      // Conditional rescale, decided for the whole wave.
      const bool grow = mx > m_run + kTau;  // false while both are -inf
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) acc[dt] *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

      // P = exp2(s*c - m), its row sum, and P^T as the bf16 B operand.
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
      bf16x8 pb[T::KT][2];
#pragma unroll
      for (int kt = 0; kt < T::KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(s[kt][r], c, -m_use));
          ls[r & 3] += e;
          pb[kt][r >> 3][r & 7] = (__bf16)e;
        }
      l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);

      // O^T += V^T P^T; V^T operands come from transpose reads of row-major V.
      const __bf16* vl = cur + T::K_ELEMS + v_lane;
#pragma unroll
      for (int kt = 0; kt < T::KT; ++kt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int dt = 0; dt < T::DT; ++dt) {
            const __bf16* p0 = vl + (kt * 32 + 16 * hh) * T::VSTR + dt * 32;
            const bf16x8 a = read_tr_pair(p0, p0 + 8 * T::VSTR);
            acc[dt] = mfma32(a, pb[kt][hh], acc[dt]);
          }
    }

    if (has_next) store_tile(nxt);
    __syncthreads();
  }

  // ---- epilogue: O = o / l in bf16, LSE = (m + log2 l) ln 2
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qrow < q_len) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    __bf16* orow = p.o + (q_row0 + qrow) * q_stride + (long)h * D;
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(acc[dt][4 * rq + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + dt * 32 + 8 * rq + 4 * g) = ov;
      }
    if (g == 0)
      p.lse[lse_base + (long)h * lse_hstride + qrow] =
          l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

thread_local int g_last_hip_error = 0;

template <int D, bool CAUSAL, bool VARLEN>
int launch_one(const Params& p, int grid, hipStream_t stream) {
  (void)hipGetLastError();  // clear a stale error so the check below is ours
  hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, VARLEN>), dim3(grid), dim3(kThreads), 0, stream,
                     p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

int dispatch(const Params& p, int d, bool causal, bool varlen, int grid, hipStream_t stream) {
  if (d == 64) {
    if (varlen) return causal ? launch_one<64, true, true>(p, grid, stream)
                              : launch_one<64, false, true>(p, grid, stream);
    return causal ? launch_one<64, true, false>(p, grid, stream)
                  : launch_one<64, false, false>(p, grid, stream);
  }
  if (varlen) return causal ? launch_one<128, true, true>(p, grid, stream)
                            : launch_one<128, false, true>(p, grid, stream);
  return causal ? launch_one<128, true, false>(p, grid, stream)
                : launch_one<128, false, false>(p, grid, stream);
}

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

int check_common(int Hq, int Hkv, int d, float scale) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_HEADS;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (!std::isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_SIZE;
  return ATTN_OK;
}

int check_buffers(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  bool need_kv) {
  if (q == nullptr || o == nullptr || lse == nullptr) return ATTN_ERR_NULL;
  if (need_kv && (k == nullptr || v == nullptr)) return ATTN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(o, 16) || !aligned(lse, 4)) return ATTN_ERR_ALIGN;
  if (need_kv && (!aligned(k, 16) || !aligned(v, 16))) return ATTN_ERR_ALIGN;
  return ATTN_OK;
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                        const int32_t* seqlens_k, void* stream) {
  if (B < 0 || Nq < 0 || Nk < 0) return ATTN_ERR_SIZE;
  int rc = check_common(Hq, Hkv, d, scale);
  if (rc != ATTN_OK) return rc;
  if (B == 0 || Nq == 0) return ATTN_OK;
  rc = check_buffers(q, k, v, o, lse, Nk > 0);
  if (rc != ATTN_OK) return rc;
  const long nqb = (Nq + kBr - 1) / kBr;
  const long grid = (long)B * Hq * nqb;
  if (grid > INT_MAX || (long)B * Nq > INT_MAX || (long)B * Nk > INT_MAX) return ATTN_ERR_TOO_LARGE;
  Params p{};
  p.q = static_cast<const __bf16*>(q);
  p.k = static_cast<const __bf16*>(k);
  p.v = static_cast<const __bf16*>(v);
  p.o = static_cast<__bf16*>(o);
  p.lse = lse;
  p.seqlens_k = seqlens_k;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.nqb = static_cast<int>(nqb);
  p.num_seqs = B;
  p.c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  return dispatch(p, d, causal != 0, false, static_cast<int>(grid),
                  static_cast<hipStream_t>(stream));
}

extern "C" int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int num_seqs, int Hq, int Hkv, int max_seqlen_q, int max_seqlen_k,
                               int d, float scale, int causal, void* stream) {
  if (num_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return ATTN_ERR_SIZE;
  int rc = check_common(Hq, Hkv, d, scale);
  if (rc != ATTN_OK) return rc;
  if (num_seqs == 0 || max_seqlen_q == 0) return ATTN_OK;
  if (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr) return ATTN_ERR_NULL;
  rc = check_buffers(q, k, v, o, lse, max_seqlen_k > 0);
  if (rc != ATTN_OK) return rc;
  const long nqb = (max_seqlen_q + kBr - 1) / kBr;
  const long grid = (long)num_seqs * Hq * nqb;
  if (grid > INT_MAX) return ATTN_ERR_TOO_LARGE;
  Params p{};
  p.q = static_cast<const __bf16*>(q);
  p.k = static_cast<const __bf16*>(k);
  p.v = static_cast<const __bf16*>(v);
  p.o = static_cast<__bf16*>(o);
  p.lse = lse;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.Nq = max_seqlen_q;
  p.Nk = max_seqlen_k;
  p.nqb = static_cast<int>(nqb);
  p.num_seqs = num_seqs;
  p.c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  return dispatch(p, d, causal != 0, true, static_cast<int>(grid),
                  static_cast<hipStream_t>(stream));
}

extern "C" const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_HEAD_DIM: return "unsupported head dimension (supported: 64, 128)";
    case ATTN_ERR_HEADS: return "bad head counts (need Hq >= 1, Hkv >= 1, Hq % Hkv == 0)";
    case ATTN_ERR_SIZE: return "negative size, or scale not finite and positive";
    case ATTN_ERR_LAUNCH: return "HIP kernel launch failed (see attn_last_hip_error)";
    case ATTN_ERR_ALIGN: return "q/k/v/o must be 16-byte aligned and lse 4-byte aligned";
    case ATTN_ERR_TOO_LARGE: return "problem too large for 32-bit grid or row indexing";
    default: return "unknown attn status";
  }
}

extern "C" int attn_last_hip_error(void) { return g_last_hip_error; }

extern "C" const char* attn_version(void) { return "0.1.0"; }
