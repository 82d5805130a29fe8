// Exact-attention backward for AMD CDNA4 (gfx950, MI355X), and its C ABI.
//
// What it computes (FlashAttention-4 (papercache summary), section 2.1, the
// backward equations): for S = scale Q K^T (masked), P = softmax(S), O = P V
// and an upstream gradient dO,
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D)  (D_i = <dO_i, O_i>),
//     dQ = scale dS K,  dK = scale dS^T Q,
// with P rebuilt from the forward's saved LSE as exp(S - LSE), so no N x N
// matrix is stored ("059 · FlashAttention" (wq-win), section 3: the backward
// recomputes probability blocks from the inputs and the saved row
// statistics).  Grouped-query heads: a KV head's gradient sums its G query
// heads.
//
// Three kernels, no atomics, deterministic:
// * bwd_preprocess: D = <dO, O> per row, and LSE in log2 units (+inf for a
//   row with no visible key, so exp2(s - lse) is 0 there), into a workspace.
// * bwd_dkdv_kernel: one workgroup of 4 waves per 128 keys of one (batch, KV
//   head); wave w owns keys 32w..32w+31 and loops over the G query heads and
//   32-row query blocks.  S = Q K^T is formed with the keys as the columns of
//   the 32x32 MFMA accumulator, so each lane holds one key and 16 queries:
//   P and dS are then B operands (k = queries) of dV^T += dO^T P and
//   dK^T += Q^T dS without leaving registers; dO^T and Q^T come from gfx950
//   transpose reads of LDS (ds_read_b64_tr_b16).  The recompute ordering of
//   FlashAttention-4 (papercache summary), section 3.2.2: iterate along the
//   KV sequence, values transposed relative to the forward.
// * bwd_dq_kernel: one workgroup of 4 waves per 128 query rows of one head;
//   the forward's orientation (S^T = K Q^T, one query per lane), with
//   dP^T = V dO^T, dS^T = P^T * (dP^T - D) and dQ^T += K^T dS^T.  dQ is
//   summed over all key blocks inside one workgroup, so it needs neither
//   atomic adds nor a reduction order (the determinism concern of
//   FlashAttention-4 (papercache summary), section 3.2.4).
//
// LDS tiles are row-major rows of d = 128 bf16 (sixteen 16-byte chunks) with
// chunk c of row r stored at position c ^ swz(r), swz(r) = 4*(r%4) + (r/4)%4.
// A 32-lane row read (32 rows, one chunk) and a transpose read (4 rows x 2
// chunks x 4 chunks per half-wave) both touch 16 distinct 16-byte bank
// groups per 16 lanes, so neither conflicts.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "attn.h"
#include "cdna4.h"

namespace {

constexpr int kD = 128;                 // head dimension of the backward kernels
constexpr int kChunks = kD / 8;         // 16-byte chunks per row
constexpr int kBwThreads = 256;         // 4 waves
constexpr int kKeysPerWg = 128;         // dK/dV kernel: keys per workgroup
constexpr int kQStep = 32;              // dK/dV kernel: query rows per step
constexpr int kQPerWg = 128;            // dQ kernel: query rows per workgroup
constexpr int kKStep = 64;              // dQ kernel: keys per step

struct BwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dout;
  const float* lse2;    // workspace: LSE * log2(e), +inf for empty rows, [B, Hq, Nq]
  const float* delta;   // workspace: <dO, O>, [B, Hq, Nq]
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  const int32_t* seqlens_k;
  int B, Hq, Hkv, G, Nq, Nk;
  int nblk;             // key blocks (dK/dV) or query blocks (dQ) per (batch, head)
  float c;              // scale * log2(e)
  float scale;
};

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Element offset of (row, chunk) in a swizzled tile.
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return row * kD + 8 * (chunk ^ swz(row));
}

// Row-operand read: lane l takes row r0 + l%32, elements 16*ks + 8*(l/32) .. +7.
__device__ __forceinline__ bf16x8 read_rows(const __bf16* t, int r0, int ks, int lane) {
  return *reinterpret_cast<const bf16x8*>(t + tile_off(r0 + (lane & 31), 2 * ks + (lane >> 5)));
}

// Transposed operand: rows r0 + {4g..4g+3} then r0 + {8+4g..8+4g+3} (g = lane/32), as the
// k-elements, for column d0 + lane%32 of the operand (d0 a multiple of 32).
__device__ __forceinline__ bf16x8 read_cols(const __bf16* t, int r0, int d0, int lane) {
  const int g = lane >> 5, m = (lane & 15) >> 2, u = lane & 3;
  const int dcol = d0 + 16 * ((lane >> 4) & 1) + 4 * u;  // first of this lane's 4 columns
  const int chunk = dcol >> 3, sub = dcol & 7;
  const int ra = r0 + 4 * g + m, rb = ra + 8;
  return read_tr_pair(t + tile_off(ra, chunk) + sub, t + tile_off(rb, chunk) + sub);
}

// Global rows [row0, row0 + rows) of a [.., stride] bf16 array -> swizzled LDS tile.
// Loads are 16 bytes per lane, row-contiguous; rows >= valid read as zero.
template <int ROWS>
struct TileCopy {
  static constexpr int kPer = ROWS * kChunks / kBwThreads;  // chunks per thread
  static_assert(kPer * kBwThreads == ROWS * kChunks, "tile split");
  u32x4 r[kPer];
  __device__ __forceinline__ void load(const __bf16* base, long stride, int valid, int tid) {
    const __amdgpu_buffer_rsrc_t res = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16*>(base), (short)0, max(valid, 0) * (int)(stride * 2), kBufferFlags);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * kBwThreads;
      const int row = c / kChunks, chunk = c % kChunks;
      r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           res, (uint32_t)(row * stride * 2 + chunk * 16), 0, 0));
    }
  }
  __device__ __forceinline__ void store(__bf16* tile, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * kBwThreads;
      *reinterpret_cast<u32x4*>(tile + tile_off(c / kChunks, c % kChunks)) = r[i];
    }
  }
};

// ---------------------------------------------------------------------------
// D = <dO, O> and LSE in log2 units, one row per 16 lanes.
__global__ __launch_bounds__(256) void bwd_preprocess(const __bf16* o, const __bf16* dout,
                                                      const float* lse, float* lse2, float* delta,
                                                      int B, int Hq, int Nq) {
  const long rows = (long)B * Nq * Hq;
  const long row = (long)blockIdx.x * 16 + (threadIdx.x >> 4);  // row of [B, Nq, Hq]
  const int sub = threadIdx.x & 15;
  float acc = 0.f;
  if (row < rows) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(o + row * kD + sub * 8);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(dout + row * kD + sub * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (row < rows && sub == 0) {
    const int h = (int)(row % Hq);
    const long bi = row / Hq;
    const int i = (int)(bi % Nq);
    const int b = (int)(bi / Nq);
    const long out = ((long)b * Hq + h) * Nq + i;
    const float l = lse[out];
    delta[out] = acc;
    lse2[out] = (l == -INFINITY) ? INFINITY : l * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dK, dV.
template <bool CAUSAL>
__global__ __launch_bounds__(kBwThreads, 1) void bwd_dkdv_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) __bf16 k_t[kKeysPerWg * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 v_t[kKeysPerWg * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 q_t[2][kQStep * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 do_t[2][kQStep * kD];
  __shared__ __attribute__((aligned(16))) float l2_t[2][kQStep];
  __shared__ __attribute__((aligned(16))) float d_t[2][kQStep];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;

  // work: (batch, KV head) units dealt round-robin to the XCDs, key blocks in order
  const int units = p.B * p.Hkv;
  const int x = blockIdx.x % kXcds, rr = blockIdx.x / kXcds;
  const int u = (rr / p.nblk) * kXcds + x;
  if (u >= units) return;
  const int kb = rr % p.nblk;
  const int b = u / p.Hkv, hkv = u % p.Hkv;
  int nk = p.Nk;
  if (p.seqlens_k != nullptr) nk = min(max(p.seqlens_k[b], 0), p.Nk);
  const int k0 = kb * kKeysPerWg;
  const long kv_stride = (long)p.Hkv * kD;
  const long q_stride = (long)p.Hq * kD;
  const __bf16* kbase = p.k + ((long)b * p.Nk + k0) * kv_stride + (long)hkv * kD;
  const __bf16* vbase = p.v + ((long)b * p.Nk + k0) * kv_stride + (long)hkv * kD;

  {  // K and V of the block, once
    TileCopy<kKeysPerWg> kc, vc;
    kc.load(kbase, kv_stride, min(nk - k0, kKeysPerWg), tid);
    vc.load(vbase, kv_stride, min(nk - k0, kKeysPerWg), tid);
    kc.store(k_t, tid);
    vc.store(v_t, tid);
  }

  const int wk0 = k0 + wave * 32;         // this wave's first key
  const int key = wk0 + (lane & 31);      // this lane's key (accumulator column)
  f32x16 dk_acc[4], dv_acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) dk_acc[t] = dv_acc[t] = f32x16{};

  // query steps: every head of the group, query blocks that can see these keys
  const int s0 = CAUSAL ? (k0 / kQStep) : 0;
  const int nsteps_h = (p.Nq + kQStep - 1) / kQStep - s0;
  const int nsteps = nk > k0 ? max(nsteps_h, 0) * p.G : 0;
  TileCopy<kQStep> qc, dc;
  float stat = 0.f;  // threads 0..63: lse2 (0..31) or delta (32..63) of one row
  auto fetch = [&](int s) {
    const int gi = s / nsteps_h, i0 = (s0 + s % nsteps_h) * kQStep;
    const int h = hkv * p.G + gi;
    const long rowbase = ((long)b * p.Nq + i0) * q_stride + (long)h * kD;
    const int valid = min(p.Nq - i0, kQStep);
    qc.load(p.q + rowbase, q_stride, valid, tid);
    dc.load(p.dout + rowbase, q_stride, valid, tid);
    if (tid < 2 * kQStep) {
      const int i = i0 + (tid & 31);
      const long sidx = ((long)b * p.Hq + h) * p.Nq + i;
      stat = (i < p.Nq) ? (tid < kQStep ? p.lse2[sidx] : p.delta[sidx])
                        : (tid < kQStep ? INFINITY : 0.f);
    }
  };
  auto put = [&](int buf) {
    qc.store(q_t[buf], tid);
    dc.store(do_t[buf], tid);
    if (tid < kQStep) l2_t[buf][tid] = stat;
    else if (tid < 2 * kQStep) d_t[buf][tid - kQStep] = stat;
  };

  if (nsteps > 0) {
    fetch(0);
    put(0);
  }
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) fetch(s + 1);
    const int i0 = (s0 + s % nsteps_h) * kQStep;
    // a wave whose keys all lie after the step's last query sees nothing (causal)
    const bool live = !CAUSAL || wk0 <= i0 + kQStep - 1;
    if (live) {
      const __bf16* qt = q_t[buf];
      const __bf16* dt = do_t[buf];
      f32x16 s_acc = {}, dp_acc = {};
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks) {
        s_acc = mfma32(read_rows(qt, 0, ks, lane), read_rows(k_t, wave * 32, ks, lane), s_acc);
        dp_acc = mfma32(read_rows(dt, 0, ks, lane), read_rows(v_t, wave * 32, ks, lane), dp_acc);
      }
      // P = exp2(s*c - lse2), dS = P (dP - D); lane: key `key`, queries 8*(r/4)+4g+r%4
      u32x4 p_pk[2], ds_pk[2];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int qi = 8 * r4 + 4 * g;  // first of this group of 4 query rows
        const float4 l2 = *reinterpret_cast<const float4*>(&l2_t[buf][qi]);
        const float4 dd = *reinterpret_cast<const float4*>(&d_t[buf][qi]);
        float pv[4], dsv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          const float lv = e == 0 ? l2.x : e == 1 ? l2.y : e == 2 ? l2.z : l2.w;
          const float dv_ = e == 0 ? dd.x : e == 1 ? dd.y : e == 2 ? dd.z : dd.w;
          const int qrow = i0 + qi + e;
          const bool vis = key < nk && (!CAUSAL || key <= qrow);
          const float pe = vis ? __builtin_amdgcn_exp2f(fmaf(s_acc[r], p.c, -lv)) : 0.f;
          pv[e] = pe;
          dsv[e] = pe * (dp_acc[r] - dv_);
        }
        const bf16x2 p01 = {(__bf16)pv[0], (__bf16)pv[1]}, p23 = {(__bf16)pv[2], (__bf16)pv[3]};
        const bf16x2 d01 = {(__bf16)dsv[0], (__bf16)dsv[1]}, d23 = {(__bf16)dsv[2], (__bf16)dsv[3]};
        p_pk[r4 >> 1][2 * (r4 & 1)] = __builtin_bit_cast(uint32_t, p01);
        p_pk[r4 >> 1][2 * (r4 & 1) + 1] = __builtin_bit_cast(uint32_t, p23);
        ds_pk[r4 >> 1][2 * (r4 & 1)] = __builtin_bit_cast(uint32_t, d01);
        ds_pk[r4 >> 1][2 * (r4 & 1) + 1] = __builtin_bit_cast(uint32_t, d23);
      }
      // dV^T += dO^T P, dK^T += Q^T dS (k = the 16 queries of slice qs)
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          dv_acc[t] = mfma32(read_cols(dt, 16 * qs, 32 * t, lane),
                             __builtin_bit_cast(bf16x8, p_pk[qs]), dv_acc[t]);
          dk_acc[t] = mfma32(read_cols(qt, 16 * qs, 32 * t, lane),
                             __builtin_bit_cast(bf16x8, ds_pk[qs]), dk_acc[t]);
        }
    }
    if (s + 1 < nsteps) put(buf ^ 1);
    __syncthreads();
  }

  // dK = scale * dK^T (transposed back), dV; lane: key `key`, d = 32t + 8*(r/4) + 4g + r%4
  if (key < p.Nk && key < k0 + kKeysPerWg) {
    __bf16* dkrow = p.dk + ((long)b * p.Nk + key) * kv_stride + (long)hkv * kD;
    __bf16* dvrow = p.dv + ((long)b * p.Nk + key) * kv_stride + (long)hkv * kD;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 a, c;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = (__bf16)(dk_acc[t][4 * r4 + e] * p.scale);
          c[e] = (__bf16)dv_acc[t][4 * r4 + e];
        }
        const int dcol = 32 * t + 8 * r4 + 4 * g;
        *reinterpret_cast<bf16x4*>(dkrow + dcol) = a;
        *reinterpret_cast<bf16x4*>(dvrow + dcol) = c;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ.
template <bool CAUSAL>
__global__ __launch_bounds__(kBwThreads, 1) void bwd_dq_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) __bf16 k_t[2][kKStep * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 v_t[2][kKStep * kD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;

  // work: (batch, KV head) units round-robin over XCDs; per unit, query blocks
  // longest first (causal), query heads of the group innermost
  const int units = p.B * p.Hkv;
  const int per_unit = p.nblk * p.G;
  const int x = blockIdx.x % kXcds, rr = blockIdx.x / kXcds;
  const int u = (rr / per_unit) * kXcds + x;
  if (u >= units) return;
  const int item = rr % per_unit;
  const int qbi = item / p.G, gi = item % p.G;
  const int qb = CAUSAL ? (p.nblk - 1 - qbi) : qbi;
  const int b = u / p.Hkv, hkv = u % p.Hkv;
  const int h = hkv * p.G + gi;
  int nk = p.Nk;
  if (p.seqlens_k != nullptr) nk = min(max(p.seqlens_k[b], 0), p.Nk);

  const long kv_stride = (long)p.Hkv * kD;
  const long q_stride = (long)p.Hq * kD;
  const int q0 = qb * kQPerWg;
  const int qrow = q0 + wave * 32 + (lane & 31);
  const int wrow0 = q0 + wave * 32;
  bf16x8 qf[kD / 16], df[kD / 16];
  const long qoff = ((long)b * p.Nq + qrow) * q_stride + (long)h * kD;
#pragma unroll
  for (int ks = 0; ks < kD / 16; ++ks) {
    qf[ks] = qrow < p.Nq ? *reinterpret_cast<const bf16x8*>(p.q + qoff + 16 * ks + 8 * g) : bf16x8{};
    df[ks] = qrow < p.Nq ? *reinterpret_cast<const bf16x8*>(p.dout + qoff + 16 * ks + 8 * g) : bf16x8{};
  }
  const long sidx = ((long)b * p.Hq + h) * p.Nq + qrow;
  const float l2 = qrow < p.Nq ? p.lse2[sidx] : INFINITY;
  const float dd = qrow < p.Nq ? p.delta[sidx] : 0.f;

  int kv_end = nk;
  if (CAUSAL) kv_end = min(nk, q0 + kQPerWg);
  const int ntiles = (kv_end + kKStep - 1) / kKStep;
  const __bf16* kbase = p.k + (long)b * p.Nk * kv_stride + (long)hkv * kD;
  const __bf16* vbase = p.v + (long)b * p.Nk * kv_stride + (long)hkv * kD;

  f32x16 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x16{};
  TileCopy<kKStep> kc, vc;
  auto fetch = [&](int j) {
    const int j0 = j * kKStep;
    kc.load(kbase + (long)j0 * kv_stride, kv_stride, min(kv_end - j0, kKStep), tid);
    vc.load(vbase + (long)j0 * kv_stride, kv_stride, min(kv_end - j0, kKStep), tid);
  };
  if (ntiles > 0) {
    fetch(0);
    kc.store(k_t[0], tid);
    vc.store(v_t[0], tid);
  }
  __syncthreads();
  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) fetch(j + 1);
    const int j0 = j * kKStep;
    const bool live = !CAUSAL || j0 <= wrow0 + 31;
    if (live) {
      const __bf16* kt = k_t[buf];
      const __bf16* vt = v_t[buf];
      u32x4 ds_pk[2][2];  // [32-key block][16-key half]
#pragma unroll
      for (int kt2 = 0; kt2 < 2; ++kt2) {
        f32x16 s_acc = {}, dp_acc = {};
#pragma unroll
        for (int ks = 0; ks < kD / 16; ++ks) {
          s_acc = mfma32(read_rows(kt, 32 * kt2, ks, lane), qf[ks], s_acc);
          dp_acc = mfma32(read_rows(vt, 32 * kt2, ks, lane), df[ks], dp_acc);
        }
        // lane: query qrow; register r: key j0 + 32*kt2 + 8*(r/4) + 4g + r%4
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float dsv[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int kk = j0 + 32 * kt2 + 8 * ((r + e) >> 2) + 4 * g + ((r + e) & 3);
            const bool vis = kk < nk && (!CAUSAL || kk <= qrow);
            const float pe = vis ? __builtin_amdgcn_exp2f(fmaf(s_acc[r + e], p.c, -l2)) : 0.f;
            dsv[e] = pe * (dp_acc[r + e] - dd);
          }
          const bf16x2 pk = {(__bf16)dsv[0], (__bf16)dsv[1]};
          ds_pk[kt2][r >> 3][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, pk);
        }
      }
      // dQ^T += K^T dS^T: A = K^T (32 d x 16 keys) from transpose reads
#pragma unroll
      for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            acc[t] = mfma32(read_cols(kt, 32 * kt2 + 16 * hh, 32 * t, lane),
                            __builtin_bit_cast(bf16x8, ds_pk[kt2][hh]), acc[t]);
    }
    if (j + 1 < ntiles) {
      kc.store(k_t[buf ^ 1], tid);
      vc.store(v_t[buf ^ 1], tid);
    }
    __syncthreads();
  }

  if (qrow < p.Nq) {
    __bf16* row = p.dq + qoff;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 a;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = (__bf16)(acc[t][4 * r4 + e] * p.scale);
        *reinterpret_cast<bf16x4*>(row + 32 * t + 8 * r4 + 4 * g) = a;
      }
  }
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) % 16) == 0; }

int launched() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    attn_detail::last_hip_error = static_cast<int>(e);
    return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

}  // namespace

extern "C" size_t attn_bwd_workspace_size(int B, int Hq, int Nq) {
  if (B <= 0 || Hq <= 0 || Nq <= 0) return 0;
  return (size_t)2 * sizeof(float) * (size_t)B * (size_t)Hq * (size_t)Nq;
}

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        void* workspace, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                        float scale, int causal, const int32_t* seqlens_k, void* stream) {
  if (B < 0 || Nq < 0 || Nk < 0) return ATTN_ERR_SIZE;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_HEADS;
  if (d != kD) return ATTN_ERR_HEAD_DIM;
  if (!std::isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_SIZE;
  if (B == 0 || (Nq == 0 && Nk == 0)) return ATTN_OK;
  const bool need_q = Nq > 0, need_k = Nk > 0;
  if ((need_k && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr)) ||
      (need_q && (q == nullptr || o == nullptr || lse == nullptr || dout == nullptr ||
                  dq == nullptr || workspace == nullptr)))
    return ATTN_ERR_NULL;
  if ((need_q && (!aligned16(q) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
                  !aligned16(workspace) || (reinterpret_cast<uintptr_t>(lse) % 4) != 0)) ||
      (need_k && (!aligned16(k) || !aligned16(v) || !aligned16(dk) || !aligned16(dv))))
    return ATTN_ERR_ALIGN;
  const long rows = (long)B * Nq * Hq;
  if (rows > INT_MAX || (long)B * Nk * Hkv > INT_MAX || (long)Nq * Hq * kD > INT_MAX / 2 ||
      (long)Nk * Hkv * kD > INT_MAX / 2)
    return ATTN_ERR_TOO_LARGE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  BwdParams p{};
  p.q = static_cast<const __bf16*>(q);
  p.k = static_cast<const __bf16*>(k);
  p.v = static_cast<const __bf16*>(v);
  p.dout = static_cast<const __bf16*>(dout);
  float* lse2 = static_cast<float*>(workspace);
  float* delta = lse2 + rows;
  p.lse2 = lse2;
  p.delta = delta;
  p.dq = static_cast<__bf16*>(dq);
  p.dk = static_cast<__bf16*>(dk);
  p.dv = static_cast<__bf16*>(dv);
  p.seqlens_k = seqlens_k;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.scale = scale;
  p.c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  const long units8 = ((long)B * Hkv + kXcds - 1) / kXcds * kXcds;
  if (need_q) {
    hipLaunchKernelGGL(bwd_preprocess, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, st,
                       static_cast<const __bf16*>(o), static_cast<const __bf16*>(dout), lse,
                       lse2, delta, B, Hq, Nq);
    if (int rc = launched()) return rc;
  }
  if (need_k) {
    p.nblk = (Nk + kKeysPerWg - 1) / kKeysPerWg;
    const long grid = units8 * p.nblk;
    if (grid > INT_MAX) return ATTN_ERR_TOO_LARGE;
    if (causal)
      hipLaunchKernelGGL(bwd_dkdv_kernel<true>, dim3((unsigned)grid), dim3(kBwThreads), 0, st, p);
    else
      hipLaunchKernelGGL(bwd_dkdv_kernel<false>, dim3((unsigned)grid), dim3(kBwThreads), 0, st, p);
    if (int rc = launched()) return rc;
  }
  if (need_q) {
    p.nblk = (Nq + kQPerWg - 1) / kQPerWg;
    const long grid = units8 * p.nblk * p.G;
    if (grid > INT_MAX) return ATTN_ERR_TOO_LARGE;
    if (causal)
      hipLaunchKernelGGL(bwd_dq_kernel<true>, dim3((unsigned)grid), dim3(kBwThreads), 0, st, p);
    else
      hipLaunchKernelGGL(bwd_dq_kernel<false>, dim3((unsigned)grid), dim3(kBwThreads), 0, st, p);
    if (int rc = launched()) return rc;
  }
  return ATTN_OK;
}

