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
// Shared CDNA4 mapping
// --------------------
// * Each wave (wave64) owns 32 query rows.  Scores are computed transposed,
//   S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: A = a 32-key slice of K read
//   from LDS, B = the wave's 32 query rows held in VGPRs for the whole
//   kernel.  In the 32x32 accumulator layout lane l holds column l%32 (one
//   query row) and 16 of the 32 key rows; lanes l and l^32 hold the other half
//   of the same row.  Row max and row sum are therefore in-lane reductions
//   plus one exchange with lane l^32 (v_permlane32_swap), and the row
//   statistics are per-lane scalars.
// * The output is accumulated transposed too, O^T += V^T P^T, with the same
//   instruction: A = a 32(d) x 16(key) slice of V^T, B = P^T taken straight
//   from the score accumulators after conversion to bf16, so P never leaves
//   registers.  The 16 keys an instruction consumes must sit in the same
//   (lane-half, slot) positions in both operands; the score layout gives
//   lane-half g the keys {4g..4g+3, 8+4g..8+4g+3} of each 16-key group.  Each
//   A operand of V^T is assembled from two gfx950 transpose reads
//   (ds_read_b64_tr_b16): in every 16-lane block, lane j addresses 4
//   consecutive d of key row j/4 and lane i receives the 4 keys of column i.
// * The d = 128 kernel (dense and block-sparse launches) runs both
//   contractions on v_mfma_f32_16x16x32_bf16 instead (a higher sustained
//   clock under the chip's power limit).  A wave's
//   32 query rows are then two 16-row blocks qb, and lane l holds rows
//   16 qb + l%16 with keys 16 kb + 4 (l/16) .. +3 of every 16-key block kb, so
//   row statistics combine lanes l, l^16, l^32 and l^48 (v_permlane16_swap,
//   then v_permlane32_swap).  A P V instruction consumes 32 keys: lane group
//   G = l/16 supplies keys 4G..4G+3 and 16+4G..16+4G+3 of them, in both
//   operands, its V^T part again two transpose reads.  In odd 4-key groups
//   the 16-wide d blocks of V are stored pairwise swapped, so the four 16-lane
//   blocks of such a read (4-key groups G = 0..3) fall on alternate LDS bank
//   halves.
// * LDS tile layouts (64 keys per tile).  K: 16-row groups, 16-byte chunk
//   major -- element offset ((row/16)*(D/8) + chunk)*128 + (row%16)*8 -- so the
//   32 lanes of a score-operand read touch 32 distinct 16-byte bank groups.
//   V: "quad sub-tiles", each 4 keys x 16 d stored as 128 contiguous bytes
//   (groups in key order, blocks in d order), so a transpose read by 32 lanes
//   covers 256 contiguous bytes.  Both are conflict-free, and a tile is
//   filled by 1 KB contiguous stores (one 16-byte chunk per lane).
// * Rows past the last valid key are read as zeros (buffer-resource range
//   check) or from a clamped valid row, and masked to -inf in the scores.
// * Conditional rescaling (FlashAttention-4 (papercache summary), section
//   3.1.4): the running max of a row is raised, and O and l rescaled, only
//   when the new block's max exceeds it by more than tau = 8 (log2 units, a
//   factor of 256); otherwise the block is accumulated against the stale max.
//   The decision is per wavefront (a ballot), so the skip is a uniform branch.
//   The final O / l and LSE = m + log2 l stay exact.
// * Softmax runs in the exp2 domain with scale*log2(e) folded into one FMA per
//   score; LSE is converted back to natural log in the epilogue.  The d = 128
//   kernel takes a tile's exponentials against the running max first and
//   computes the row maxima only when some lane's partial sum shows that the
//   rescale might fire (a sum above 2^tau); the results are those of the
//   max-first step bit for bit.
// * O leaves through LDS: each wave writes its normalised rows there and
//   stores them whole, 16 bytes per lane, instead of the 8-byte pieces of 32
//   rows that its accumulator layout holds.
// * Causal: key blocks past the query block's last row are never visited;
//   masks are applied only on blocks that cross the diagonal or the key tail.
// * Grid order (decode_work): (batch or sequence, KV head) units are dealt
//   round-robin to the 8 XCDs, each XCD running its units one after another,
//   query blocks longest first under the causal mask and the query heads of
//   the KV group innermost.  The workgroups resident on one XCD thus read the
//   same K/V from its L2, and every XCD gets a like share of every batch
//   element.  Packed batches can also be taken in the longest-first sequence
//   order written by varlen_plan_kernel (longest-processing-time-first
//   scheduling, head grouping and the varlen batch map of FlashAttention-4
//   (papercache summary), section 3.3).
//
// Two kernels
// -----------
// * d = 128: attn_fwd_pp_kernel, 8 waves / 256 query rows per workgroup (of
//   up to 8 query heads of one KV group, 256 / heads rows each) in two groups
//   of four; the two waves sharing a SIMD belong to different
//   groups and run half a period apart, so one feeds the matrix core (scores
//   of tile j, then P V of tile j-1) while the other computes its softmax --
//   the CDNA form of the ping-pong of FlashAttention-4 (papercache summary),
//   section 3.1.2.  One workgroup barrier per half period.  K/V tiles move
//   global -> VGPRs -> LDS (16-byte loads, one tile per group per period,
//   double-buffered), the LDS stores spread over the MFMA phase.  When a
//   unit has an even number of query blocks and at most 8192 keys (and the
//   launch is not block-sparse) a workgroup runs two of them, the i-th
//   longest and the i-th shortest, back to back.  d = 128 launches (dense
//   and block-sparse) run it on 16x16x32 MFMAs, (192, 128) ones on 32x32x16.
// * d = 64: attn_fwd_kernel, 4 waves / 128 query rows per workgroup, each
//   wave interleaving its own softmax with its MFMAs slice by slice; K/V tiles
//   move global -> LDS directly (buffer_load ... lds), K two tiles ahead.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "attn.h"
#include "cdna4.h"

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBr = kWaves * kRowsPerWave;  // query rows per workgroup

template <int D>
struct Tile {
  static constexpr int BC = 64;                    // keys per step
  static constexpr int KT = BC / 32;               // 32-key MFMA blocks per step
  static constexpr int DT = D / 32;                // 32-wide d blocks of O^T
  static constexpr int KS = D / 16;                // 16-deep d slices of S^T
  static constexpr int QUAD = 4 * D;               // V elements per 4-key group in LDS
  static constexpr int K_ELEMS = BC * D;           // one K tile
  static constexpr int V_ELEMS = BC * D;           // one V tile
  static constexpr int CHUNKS = BC * D / 8 / kThreads;  // 16-byte chunks per thread per tile
  static_assert(CHUNKS * kThreads * 8 == BC * D, "tile split");
};

constexpr float kTau = 8.0f;  // conditional-rescale threshold, log2 units
// Iteration kinds of the d = 64 kernel (which parts are fixed at compile time).
constexpr int kGeneric = 0, kSteady = 1, kFirst = 2, kLast = 3;
constexpr float kTwoPowTau = 256.0f;  // 2^kTau

// Race check.  A library built with -DATTN_FORCE_SAFE=1 keeps every
// arithmetic step and its order but synchronises conservatively: the two
// wave groups of the ping-pong kernel run in lockstep instead of half a
// period apart (every LDS buffer is then written and read in different
// phases of all waves alike), every LDS store and global load is waited for
// at once and followed by a workgroup barrier, and the d = 64 kernel waits for
// its tile DMA before computing.  Its outputs must equal the tuned build's
// bit for bit; a difference exposes a missing wait or barrier.
#ifndef ATTN_FORCE_SAFE
#define ATTN_FORCE_SAFE 0
#endif
constexpr bool kForceSafe = ATTN_FORCE_SAFE != 0;

// The d = 128 forward (dense and block-sparse) on v_mfma_f32_16x16x32_bf16
// (1, the default) or on v_mfma_f32_32x32x16_bf16 (0), the shape the
// (192, 128) kernel always uses: with 16x16x32 it would exceed 256 VGPRs and
// spill.
// Under the chip's power limit the smaller shape holds a higher clock (fewer
// accumulator registers read per FLOP), at the price of twice as many MFMA
// issues and row statistics spread over four lanes instead of two.
#ifndef ATTN_PP_MFMA16
#define ATTN_PP_MFMA16 1
#endif
constexpr bool kPpMfma16 = ATTN_PP_MFMA16 != 0;

// Exponentials of the d = 128 softmax evaluated on the FMA pipe (exp2_poly)
// instead of v_exp_f32: this many of the 32 per lane and key tile (0, 4, 8
// or 16; element e of a lane's tile when e % 8 < count / 4).
#ifndef ATTN_EXP2_POLY
#define ATTN_EXP2_POLY 0
#endif
constexpr int kExp2Poly = ATTN_EXP2_POLY;
static_assert(kExp2Poly == 0 || kExp2Poly == 4 || kExp2Poly == 8 || kExp2Poly == 16, "exp2 split");

struct Params {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  const int32_t* seqlens_k;  // padded form, may be null
  const int32_t* cu_q;       // packed form
  const int32_t* cu_k;
  const int32_t* seq_order;  // packed form: virtual -> actual sequence, may be null
  int Hq, Hkv, G;
  int Nq, Nk;  // packed form: max_seqlen_q, max_seqlen_k
  int nqb;     // query blocks per (sequence, head)
  int items;   // work items (the ids decode_work reads)
  int paired;  // 1: a ping-pong workgroup runs two items of one unit (the i-th longest and shortest)
  int pack;    // query heads of one KV group per workgroup (1, 2, 4 or 8; 1 unless d = 128)
  int num_seqs;
  float c;    // |scale| * log2(e) (log2(e) when scale == 0)
  int qsign;  // sign of scale: 1, -1 (query fragments negated) or 0 (query fragments zeroed)
  const uint8_t* block_mask;  // block-sparse form: [mask_heads, nbq, nbk] of 128 x 128 blocks
  int mask_heads, nbq, nbk;
};

constexpr int kSparseBlock = 128;      // block-sparse mask granularity (rows and keys)
constexpr int kMaxSparseTiles = 4096;  // key tiles a block-sparse launch may visit (Nk <= 262144)

// Work decode.  A unit is one (batch element or sequence, KV head) pair,
// u = b * Hkv + hkv.  Units are dealt round-robin to the 8 XCDs (the hardware
// sends workgroup id w to XCD w % 8): XCD x runs units x, x+8, x+16, ... in
// that order, each unit's items back to back -- query blocks longest first
// under the causal mask, the query heads of the KV group innermost.  So the
// workgroups resident on one XCD stream the same K/V through its L2, and every
// XCD gets a like share of every batch element, also when their lengths
// differ (longest-processing-time-first order of FlashAttention-4
// (papercache summary), section 3.3).  An id is a work item; a workgroup of
// XCD x takes only ids x + 8 r (one id, its own, when the grid has one
// workgroup per item).  The ids cover ceil(units / 8) * 8 units; ids past the
// last unit are padding.
struct WorkItem {
  int b, hkv, qb, gi;
  bool valid;
};

__device__ __forceinline__ WorkItem decode_work(const Params& p, bool causal, int id) {
  const int units = p.num_seqs * p.Hkv;
  const int groups = p.G / p.pack;  // workgroups per query block of a unit
  const int per_unit = p.nqb * groups;
  const int x = id % kXcds;
  const int r = id / kXcds;
  const int u = (r / per_unit) * kXcds + x;
  const int item = r % per_unit;
  const int qbi = item / groups;
  WorkItem w;
  w.valid = u < units;
  w.b = u / p.Hkv;
  w.hkv = u % p.Hkv;
  w.gi = (item % groups) * p.pack;  // first query head of the group this workgroup takes
  w.qb = causal ? (p.nqb - 1 - qbi) : qbi;
  return w;
}

// The sign of the scale, applied to the query fragments once per work item.
// The kernels multiply scores by c = |scale| * log2(e) > 0 and take row maxima
// of the raw MFMA results, which is right only for a positive factor; with
// the queries negated the raw results are -<q, k>, and -<q, k> * |scale| is
// scale * <q, k>.  Negating bf16 is exact and fp32 accumulation rounds
// symmetrically, so a negative scale gives bitwise the result of -scale on
// negated queries.  With scale == 0 the queries are zeroed: every visible
// score is exactly 0 and masked keys stay at -inf for any c > 0.
template <int N>
__device__ __forceinline__ void apply_qsign(bf16x8 (&qf)[N], int qsign) {
  if (qsign > 0) return;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const u32x4 x = __builtin_bit_cast(u32x4, qf[i]);
    qf[i] = qsign == 0 ? bf16x8{} : __builtin_bit_cast(bf16x8, x ^ 0x80008000u);
  }
}

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(Params p) {
  using T = Tile<D>;
  // Four LDS tiles, as distinct arrays: with the tile parity known at compile
  // time the compiler can tell a DMA write to one tile from a read of another
  // and does not make the read wait for the DMA.
  __shared__ __attribute__((aligned(1024))) __bf16 k_lds0[T::K_ELEMS];
  __shared__ __attribute__((aligned(1024))) __bf16 k_lds1[T::K_ELEMS];
  __shared__ __attribute__((aligned(1024))) __bf16 v_lds0[T::V_ELEMS];
  __shared__ __attribute__((aligned(1024))) __bf16 v_lds1[T::V_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int g = lane >> 5;

  // ---- work item (see decode_work)
  const WorkItem wi = decode_work(p, CAUSAL, blockIdx.x);
  if (!wi.valid) return;  // grid padding; uniform over the workgroup
  const int b = (VARLEN && p.seq_order != nullptr)
                    ? min(max(p.seq_order[wi.b], 0), p.num_seqs - 1)
                    : wi.b;
  const int hkv = wi.hkv, qb = wi.qb, gi = wi.gi;
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
  const int wrow0 = q0 + wave * kRowsPerWave;
  const int wrow_last = wrow0 + kRowsPerWave - 1;
  const int qrow = wrow0 + l32;
  bf16x8 qf[T::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks)
    qf[ks] = qrow < q_len
                 ? *reinterpret_cast<const bf16x8*>(qbase + qrow * q_stride + ks * 16 + 8 * g)
                 : bf16x8{};
  apply_qsign(qf, p.qsign);

  // Keys this workgroup needs: all visible keys of its rows.
  int kv_end = nk;
  if (CAUSAL) kv_end = min(nk, min(q0 + kBr, q_len));
  const int n_tiles = (kv_end + T::BC - 1) / T::BC;

  // ---- global -> LDS tile loads (buffer_load ... lds, 16 bytes per lane).
  // Instruction i of wave w fills the 1 KB of LDS slots [(i*kWaves + w)*64, +64)
  // of the tile, one 16-byte slot per lane; each lane fetches the global
  // chunk that belongs in its slot under the tile's LDS layout:
  //   K, 16-row groups: slot c holds row 16*(c / (16*D/8)) + c%16, 16-byte
  //     column (c % (16*D/8)) / 16;
  //   V, quad sub-tiles: slot c holds key 4*(c / (D/2)) + (c%8)/2, columns
  //     16*((c % (D/2)) / 8) + 8*(c%2) .. +7.
  const uint32_t row_bytes = static_cast<uint32_t>(kv_stride) * 2u;
  auto k_slot = [&](int c, int* row, int* colb) __attribute__((always_inline)) {
    const int rem16 = c % (16 * (D / 8));
    *row = 16 * (c / (16 * (D / 8))) + rem16 % 16;
    *colb = (rem16 / 16) * 16;
  };
  auto v_slot = [&](int c, int* row, int* colb) __attribute__((always_inline)) {
    const int w = c % (D / 2);
    *row = 4 * (c / (D / 2)) + (w % 8) / 2;
    *colb = (16 * (w / 8) + 8 * (w % 2)) * 2;
  };
  uint32_t kgoff[T::CHUNKS], vgoff[T::CHUNKS];  // byte offsets within a full tile
#pragma unroll
  for (int i = 0; i < T::CHUNKS; ++i) {
    const int c = (i * kWaves + wave) * 64 + lane;
    int row, colb;
    k_slot(c, &row, &colb);
    kgoff[i] = row * row_bytes + colb;
    v_slot(c, &row, &colb);
    vgoff[i] = row * row_bytes + colb;
  }
  // Rows at or past kv_end (only in the last tile) are fetched from row
  // kv_end - 1 (valid memory) and masked out of the scores, so no lane ever
  // multiplies uninitialised LDS.
  auto issue_tile = [&](const __bf16* base, __bf16* dst, const uint32_t* goff, bool is_v,
                        int kv0) __attribute__((always_inline)) {
    const int nrows = min(kv_end - kv0, T::BC);
    const __amdgpu_buffer_rsrc_t res = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16*>(base + kv0 * kv_stride), (short)0, nrows * (int)row_bytes,
        kBufferFlags);
#pragma unroll
    for (int i = 0; i < T::CHUNKS; ++i) {
      uint32_t off = goff[i];
      if (nrows < T::BC) {
        int row, colb;
        const int c = (i * kWaves + wave) * 64 + lane;
        if (is_v) v_slot(c, &row, &colb); else k_slot(c, &row, &colb);
        off = (uint32_t)min(row, nrows - 1) * row_bytes + (uint32_t)colb;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          res, (__attribute__((address_space(3))) void*)(dst + (i * kWaves + wave) * 512), 16,
          off, 0, 0, 0);
    }
  };

  // ---- per-lane LDS read offsets (elements)
  // K (A operand of S^T): row kt*32 + l32, 16-byte column 2ks + g.
  const int k_lane = ((l32 >> 4) * (D / 8) + g) * 128 + (l32 & 15) * 8;
  // V (transpose reads): key group g of each 8-key half, 16-column block
  // (l/16)%2 of each 32-wide d block, row (l%16)/4, columns 4*(l%4)..+3.
  const int v_lane = g * T::QUAD + ((lane >> 4) & 1) * 64 + ((lane & 15) >> 2) * 16 + 4 * (lane & 3);

  const float c = p.c;
  // A wave skips key tiles lying wholly above its rows (causal).
  auto active = [&](int tile) __attribute__((always_inline)) { return !CAUSAL || tile * T::BC <= wrow_last; };
  auto needs_mask = [&](int tile) __attribute__((always_inline)) {
    const int kv0 = tile * T::BC;
    return (kv0 + T::BC > nk) || (CAUSAL && kv0 + T::BC - 1 > wrow0);
  };

  // ---- per-lane state: S^T of one tile (32 keys x 2 blocks of this lane's
  // row), P^T of one tile as bf16 MFMA operands, O^T, row statistics.
  f32x16 sv[T::KT];
  u32x4 pv_op[T::KT][2];  // P^T operands, bf16 pairs packed in 32-bit words
  f32x16 acc[T::DT];
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt) acc[dt] = f32x16{};
  float m_run = -INFINITY;  // running max, log2 domain (scores times scale*log2 e)
  float l_run = 0.f;        // this lane's half of the running sum
  float m_use = 0.f;        // m_run, or 0 while it is -inf (no visible key yet)
  float alpha = 1.f;
  bool rescale_o = false;   // wave-uniform: O must be multiplied by alpha

  // ---- slice plan of one iteration (tile j; one MFMA per slice).  Slices
  // 0..kPv-1 are the P V MFMAs of tile j-1, slices kPv.. the score MFMAs of
  // tile j+1 (key block 0, then 1).  The softmax of tile j rides along:
  //   P V of key block 0   | row max of S_j
  //   P V of key block 1   | rescale decision; exponentials of S_j block 0 -> P block 0
  //   scores, key block 0  | exponentials of S_j block 1 -> P block 1
  //   scores, key block 1  |
  // so every read of S_j / P_{j-1} precedes, in program order, the write of
  // S_{j+1} / P_j to the same registers, and no second copy is kept.  Slices
  // are separated by scheduling barriers (source order is the schedule) and
  // each one reads the LDS operand of the next ahead of use.
  constexpr int kPv = T::KT * 2 * T::DT;  // P V slices (one V operand each)
  constexpr int kS = T::KT * T::KS;       // score slices (one K operand each)
  constexpr int kSlices = kPv + kS;
  constexpr int kDecide = kPv / 2;        // first slice of P V key block 1
  constexpr int kAhead = 3;               // LDS read lookahead, in slices
  static_assert(T::KT == 2 && kDecide >= 2 && 32 % kDecide == 0, "slice plan");
  auto load_operand = [&](int sl, const __bf16* vb, const __bf16* kb) __attribute__((always_inline)) -> bf16x8 {
    if (sl < kPv) {
      const int kt = sl / (2 * T::DT), hh = (sl / T::DT) % 2, dt = sl % T::DT;
      const __bf16* p0 = vb + v_lane + (8 * kt + 4 * hh) * T::QUAD + dt * 128;
      return read_tr_pair(p0, p0 + 2 * T::QUAD);
    }
    const int kt = (sl - kPv) / T::KS, ks = (sl - kPv) % T::KS;
    return *reinterpret_cast<const bf16x8*>(kb + k_lane + (2 * kt * (D / 8) + 2 * ks) * 128);
  };
  // Exponentials of S_j key block kt, score registers [r0, r1).  The packed
  // bf16 pair and the partial row sums are pinned with an empty asm so the
  // compiler cannot sink this work out of its slice towards the next
  // iteration's use.
  auto exps = [&](int kt, int r0, int r1, float* ls, const float m_use) __attribute__((always_inline)) {
#pragma unroll
    for (int r = r0; r < r1; r += 2) {
      const float e0 = __builtin_amdgcn_exp2f(fmaf(sv[kt][r], c, -m_use));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(sv[kt][r + 1], c, -m_use));
      ls[0] += e0;
      ls[1] += e1;
      const bf16x2 pk = {(__bf16)e0, (__bf16)e1};
      uint32_t u = __builtin_bit_cast(uint32_t, pk);
      asm volatile("" : "+v"(u), "+v"(ls[0]), "+v"(ls[1]));
      pv_op[kt][r >> 3][(r & 7) >> 1] = u;
    }
  };
  // Keys below key_lim are visible to this lane's row; each score position
  // is a compile-time offset from the lane's first key, so the mask is one
  // compare per score.
  const int key_lim = CAUSAL ? min(nk, qrow + 1) : nk;
  auto apply_mask = [&](int tile) __attribute__((always_inline)) {
    const int t = key_lim - tile * T::BC - 4 * g;
#pragma unroll
    for (int kt = 0; kt < T::KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (!(kt * 32 + 8 * (r >> 2) + (r & 3) < t)) sv[kt][r] = -INFINITY;
  };
  // One iteration.  vb: LDS tile of V_{j-1}; kb: LDS tile of K_{j+1}.  The
  // kind (compile-time) fixes which parts run:
  //   kSteady: a predecessor and an active successor exist and tile j needs
  //     no mask, so every predicate folds to true;
  //   kFirst: j = 0 with an active successor (no P V);
  //   kLast: tile j is active and needs no mask, its predecessor exists, its
  //     successor does not (no scores);
  //   kGeneric: every predicate at run time.
  // kFirst and kGeneric mask tile j when it needs it.
  auto iteration = [&](int j, const __bf16* vb, const __bf16* kb, auto kind_tag) __attribute__((always_inline)) {
    constexpr int KIND = decltype(kind_tag)::value;
    constexpr bool FAST = KIND == kSteady || KIND == kLast;  // no mask
    const bool do_pv = KIND == kSteady || KIND == kLast || (KIND == kGeneric && j >= 1 && active(j - 1));
    const bool do_sm = KIND != kGeneric || active(j);
    const bool do_s = KIND == kSteady || KIND == kFirst ||
                      (KIND == kGeneric && j + 1 < n_tiles && active(j + 1));
    if (!FAST && do_sm && needs_mask(j)) apply_mask(j);
    float m0 = -INFINITY, m1 = -INFINITY;
    float ls[2] = {0.f, 0.f};
    // LDS operands are read kAhead slices before their MFMA.
    bf16x8 opnd[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      opnd[i] = bf16x8{};
      if (i < kPv ? do_pv : do_s) opnd[i] = load_operand(i, vb, kb);
    }
#pragma unroll
    for (int sl = 0; sl < kSlices; ++sl) {
      const bf16x8 a = opnd[sl % kAhead];
      const int nx = sl + kAhead;
      if (nx < kSlices && (nx < kPv ? do_pv : do_s)) opnd[sl % kAhead] = load_operand(nx, vb, kb);
      if (sl < kPv) {
        const int kt = sl / (2 * T::DT), hh = (sl / T::DT) % 2, dt = sl % T::DT;
        if (do_pv) acc[dt] = mfma32(a, __builtin_bit_cast(bf16x8, pv_op[kt][hh]), acc[dt]);
      } else {
        const int kt = (sl - kPv) / T::KS, ks = (sl - kPv) % T::KS;
        if (do_s) sv[kt] = mfma32(a, qf[ks], ks == 0 ? f32x16{} : sv[kt]);
      }
      if (do_sm) {
        if (sl < kDecide) {
          // row max over the 32 scores of this lane, spread over kDecide slices
          constexpr int per = 32 / kDecide;
          const int e0 = sl * per;
#pragma unroll
          for (int e = e0; e < e0 + per; e += 4) {
            m0 = max3f(m0, sv[e / 16][e % 16], sv[e / 16][e % 16 + 1]);
            m1 = max3f(m1, sv[e / 16][e % 16 + 2], sv[e / 16][e % 16 + 3]);
          }
        } else if (sl == kDecide) {
          // Conditional rescale (tau), decided for the whole wave; without
          // it alpha would be exactly 1, so nothing is computed.
          const float mx = pair_max(max3f(m0, m1, -INFINITY)) * c;
          if (__builtin_amdgcn_ballot_w64(mx > m_run + kTau) != 0) {
            const float m_new = fmaxf(m_run, mx);
            alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
            m_use = (m_new == -INFINITY) ? 0.f : m_new;
            rescale_o = true;
          }
        } else if (sl < kPv) {
          // exponentials of key block 0 over slices kDecide+1 .. kPv-1
          constexpr int nsl = kPv - kDecide - 1;
          const int i = sl - kDecide - 1;
          exps(0, 2 * ((i * 8) / nsl), 2 * (((i + 1) * 8) / nsl), ls, m_use);
        } else if (sl < kPv + T::KS) {
          // exponentials of key block 1 over the score slices of key block 0
          const int i = sl - kPv;
          exps(1, 2 * ((i * 8) / T::KS), 2 * (((i + 1) * 8) / T::KS), ls, m_use);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (do_sm) l_run += ls[0] + ls[1];
    // The deferred O rescale: after the P V of tile j-1 (relative to the old
    // max), before the P V of tile j.
    if (rescale_o) {
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt) acc[dt] *= alpha;
      rescale_o = false;
    }
  };
  // P V of the last tile (its V was loaded during the last iteration).
  auto last_pv = [&](const __bf16* vb) __attribute__((always_inline)) {
#pragma unroll
    for (int sl = 0; sl < kPv; ++sl) {
      const int kt = sl / (2 * T::DT), hh = (sl / T::DT) % 2, dt = sl % T::DT;
      acc[dt] = mfma32(load_operand(sl, vb, vb), __builtin_bit_cast(bf16x8, pv_op[kt][hh]), acc[dt]);
    }
  };

  // ---- prologue: K_0, K_1 in LDS, scores of tile 0
  if (n_tiles > 0) issue_tile(kbase, k_lds0, kgoff, false, 0);
  if (n_tiles > 1) issue_tile(kbase, k_lds1, kgoff, false, T::BC);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (n_tiles > 0 && active(0)) {
#pragma unroll
    for (int sl = kPv; sl < kSlices; ++sl) {
      const int kt = (sl - kPv) / T::KS, ks = (sl - kPv) % T::KS;
      sv[kt] = mfma32(load_operand(sl, v_lds0, k_lds0), qf[ks], ks == 0 ? f32x16{} : sv[kt]);
    }
  }
  __syncthreads();  // every wave is done with K_0 before K_2 overwrites it

  // ---- iterations.  Iteration j loads K_{j+2} into the tile K_j used and
  // V_j into the tile V_{j-2} used, reads V_{j-1} and K_{j+1}.
  auto step_static = [&](int j, auto par, auto kind_tag) __attribute__((always_inline)) {
    constexpr bool P = decltype(par)::value;  // parity of j
    __bf16* kw = P ? k_lds1 : k_lds0;
    __bf16* vw = P ? v_lds1 : v_lds0;
    const __bf16* kr = P ? k_lds0 : k_lds1;
    const __bf16* vr = P ? v_lds0 : v_lds1;
    if (j + 2 < n_tiles) issue_tile(kbase, kw, kgoff, false, (j + 2) * T::BC);
    issue_tile(vbase, vw, vgoff, true, j * T::BC);
    if constexpr (kForceSafe) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    iteration(j, vr, kr, kind_tag);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  auto step_dynamic = [&](int j) __attribute__((always_inline)) {  // buffers chosen at run time (generic iterations)
    const bool P = j & 1;
    if (j + 2 < n_tiles) issue_tile(kbase, P ? k_lds1 : k_lds0, kgoff, false, (j + 2) * T::BC);
    issue_tile(vbase, P ? v_lds1 : v_lds0, vgoff, true, j * T::BC);
    if constexpr (kForceSafe) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    iteration(j, P ? v_lds0 : v_lds1, P ? k_lds0 : k_lds1, std::integral_constant<int, kGeneric>{});
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // Steady-state iterations form one contiguous range [1, j_hi) per wave;
  // it runs unrolled by two so that the tile parity (hence every LDS buffer)
  // is a compile-time choice.  Every iteration has exactly one barrier, so
  // all waves agree on the barrier count.
  int j_hi = 1;
  while (j_hi + 1 < n_tiles && active(j_hi + 1) && !needs_mask(j_hi)) ++j_hi;
  // The first iteration, and the workgroup's last one where this wave is
  // active there and the tile is unmasked, run with compile-time buffers and
  // parts; the other iterations past the steady range (masked tiles, waves
  // whose rows end earlier, single-tile items) run generic.
  if (n_tiles > 1 && active(1)) {
    step_static(0, std::false_type{}, std::integral_constant<int, kFirst>{});
  } else if (n_tiles > 0) {
    step_dynamic(0);
  }
  int j = 1;
  for (; j + 1 < j_hi; j += 2) {
    step_static(j, std::true_type{}, std::integral_constant<int, kSteady>{});
    step_static(j + 1, std::false_type{}, std::integral_constant<int, kSteady>{});
  }
  if (j < j_hi) step_static(j++, std::true_type{}, std::integral_constant<int, kSteady>{});
  for (j = max(j, 1); j < n_tiles - 1; ++j) step_dynamic(j);
  if (j == n_tiles - 1 && j >= 1) {
    if (!active(j) || needs_mask(j)) step_dynamic(j);
    else if (j & 1) step_static(j, std::true_type{}, std::integral_constant<int, kLast>{});
    else step_static(j, std::false_type{}, std::integral_constant<int, kLast>{});
  }
  if (n_tiles > 0 && active(n_tiles - 1)) last_pv(((n_tiles - 1) & 1) ? v_lds1 : v_lds0);

  // ---- epilogue: O = o / l in bf16, LSE = (m + log2 l) ln 2.  O leaves
  // through LDS as in the ping-pong kernel: each wave writes its 32 x D block
  // row-major (16-byte chunk c of row r at c XOR (r % (D/8))) into half of a
  // K buffer, which no wave reads after the last barrier (the final P V reads
  // V only), and stores whole rows with 16-byte stores.
  constexpr int kOChunks = D / 8;
  static_assert(64 % kOChunks == 0 && kRowsPerWave % (64 / kOChunks) == 0, "O row passes");
  static_assert(kWaves == 4 && 2 * kRowsPerWave * D <= T::K_ELEMS, "O blocks fit the K buffers");
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  __bf16* const ost = (wave < 2 ? k_lds0 : k_lds1) + (wave & 1) * (kRowsPerWave * D);
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      bf16x4 ov;
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(acc[dt][4 * rq + e] * inv);
      const int chk = (dt * 4 + rq) ^ (l32 % kOChunks);  // columns dt*32 + 8 rq .. +7
      *reinterpret_cast<bf16x4*>(ost + l32 * D + chk * 8 + 4 * g) = ov;
    }
  // the wave's LDS writes precede its reads of other lanes' data
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  __bf16* const obase = p.o + (q_row0 + wrow0) * q_stride + (long)h * D;
  constexpr int kRowsPerPass = 64 / kOChunks;
  const int cc = lane % kOChunks;
#pragma unroll
  for (int i = 0; i < kRowsPerWave / kRowsPerPass; ++i) {
    const int r = i * kRowsPerPass + lane / kOChunks;
    const u32x4 ov = *reinterpret_cast<const u32x4*>(ost + r * D + (cc ^ (r % kOChunks)) * 8);
    if (wrow0 + r < q_len) *reinterpret_cast<u32x4*>(obase + r * q_stride + cc * 8) = ov;
  }
  if (qrow < q_len && g == 0)
    p.lse[lse_base + (long)h * lse_hstride + qrow] =
        l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// Ping-pong forward: 8 waves per workgroup in two groups of 4.  The two waves
// that share a SIMD belong to different groups.  Each wave alternates an MFMA
// phase (scores of tile j, then P V of tile j-1) and a VALU phase (softmax of
// tile j); group 1 runs half a period behind group 0, so while one wave of a
// SIMD feeds the matrix core the other computes its exponentials.  One
// workgroup barrier per half period keeps the groups in step.
constexpr int kPpWaves = 8;
constexpr int kPpThreads = 64 * kPpWaves;
constexpr int kPpBr = kPpWaves * kRowsPerWave;  // 256 query rows per workgroup

template <int DQK, int DV, bool CAUSAL, bool VARLEN, bool SPARSE = false, bool M16 = false>
__global__ __launch_bounds__(kPpThreads, 1) void attn_fwd_pp_kernel(Params p) {
  // Q and K rows have DQK elements, V and O rows DV (FlashAttention-4's (192, 128) shape).
  using T = Tile<DQK>;   // key tiles, score slices
  using TV = Tile<DV>;   // value tiles, output blocks
  // M16: scores and P V on v_mfma_f32_16x16x32_bf16.  A lane then holds two
  // query rows (16 qb + l%16, qb = 0, 1) and 16 keys of each per tile, whose
  // row statistics combine the four lanes l, l^16, l^32, l^48.
  static_assert(!M16 || (DQK % 32 == 0 && DV % 16 == 0), "16x16x32 shapes");
  constexpr int QB = M16 ? 2 : 1;            // query rows per lane
  constexpr int KS16 = DQK / 32;             // 32-deep d steps of a 16x16x32 score
  constexpr int DB16 = DV / 16;              // 16-wide d blocks of a 16x16x32 O^T
  using SV = std::conditional_t<M16, f32x4, f32x16>;
  constexpr int NSV = M16 ? 4 * QB : T::KT;      // score accumulators (M16: [key block][row])
  constexpr int NACC = M16 ? DB16 * QB : TV::DT;  // O^T accumulators (M16: [d block][row])
  // 16-byte chunks per thread per tile (one group of 4 waves moves a tile)
  constexpr int CHK = T::BC * DQK / 8 / (kPpThreads / 2);
  constexpr int CHV = T::BC * DV / 8 / (kPpThreads / 2);
  constexpr int CH = CHK > CHV ? CHK : CHV;
  static_assert(CHK * kPpThreads * 8 == 2 * T::BC * DQK && CHV * kPpThreads * 8 == 2 * T::BC * DV,
                "tile split");
  constexpr int kOChunks = DV / 8;  // 16-byte chunks of an O row
  static_assert(64 % kOChunks == 0 && kRowsPerWave % (64 / kOChunks) == 0, "O row passes");
  static_assert(2 * kRowsPerWave * DV <= T::K_ELEMS && 2 * kRowsPerWave * DV <= TV::V_ELEMS,
                "two waves' O blocks fit one K or V buffer");
  __shared__ __attribute__((aligned(1024))) __bf16 k_lds0[T::K_ELEMS];
  __shared__ __attribute__((aligned(1024))) __bf16 k_lds1[T::K_ELEMS];
  __shared__ __attribute__((aligned(1024))) __bf16 v_lds0[TV::V_ELEMS];
  __shared__ __attribute__((aligned(1024))) __bf16 v_lds1[TV::V_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int chunk = 2 * (wave & 3) + grp;  // 32-row chunk of the query block
  const int l32 = lane & 31;
  const int g = lane >> 5;

  __shared__ int tile_list[SPARSE ? kMaxSparseTiles : 1];  // block-sparse work list
  __shared__ int wave_count[SPARSE ? kPpWaves : 1];

  // One work item: a query block of P query heads of one (sequence, KV head)
  // unit.  Returns at the same point in every wave.
  auto run_item = [&](const int item) __attribute__((always_inline)) {
    // ---- work item (see decode_work)
    const WorkItem wi = decode_work(p, CAUSAL, item);
    if (!wi.valid) return;  // grid padding; uniform over the workgroup
    const int b = (VARLEN && p.seq_order != nullptr)
                      ? min(max(p.seq_order[wi.b], 0), p.num_seqs - 1)
                      : wi.b;
    const int hkv = wi.hkv, qb = wi.qb, gi = wi.gi;
    // The workgroup takes P query heads of the KV group, 256 / P rows of each:
    // chunk c holds rows (c % cph) * 32 .. +31 of head gi + c / cph.  The two
    // waves of a SIMD (chunks 2s, 2s+1) always share their causal extent.
    const int P = SPARSE ? 1 : p.pack;
    const int cph = kPpWaves / P;               // 32-row chunks per head
    const int rows_h = kRowsPerWave * cph;      // query rows per head
    const int h = hkv * p.G + gi + chunk / cph;

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
    const int q0 = qb * rows_h;
    if (q0 >= q_len) return;  // uniform over the workgroup, before any barrier

    const long q_stride = (long)p.Hq * DQK;
    const long o_stride = (long)p.Hq * DV;
    const long k_stride = (long)p.Hkv * DQK;
    const long v_stride = (long)p.Hkv * DV;
    const __bf16* qbase = p.q + q_row0 * q_stride + (long)h * DQK;
    const __bf16* kbase = p.k + k_row0 * k_stride + (long)hkv * DQK;
    const __bf16* vbase = p.v + k_row0 * v_stride + (long)hkv * DV;

    const int wrow0 = q0 + (chunk % cph) * kRowsPerWave;
    const int qrow = wrow0 + l32;
    // query row qb of this lane (M16; else its one row)
    auto qrow_of = [&](int qb) __attribute__((always_inline)) {
      return M16 ? wrow0 + 16 * qb + (lane & 15) : qrow;
    };
    bf16x8 qf[T::KS];  // M16: qf[qb * KS16 + s] holds d 32 s + 8 (l/16) .. +7
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      if constexpr (M16) {
        const int qr = qrow_of(ks / KS16);
        qf[ks] = qr < q_len ? *reinterpret_cast<const bf16x8*>(qbase + (long)qr * q_stride +
                                                              (ks % KS16) * 32 + 8 * (lane >> 4))
                            : bf16x8{};
      } else {
        qf[ks] = qrow < q_len
                     ? *reinterpret_cast<const bf16x8*>(qbase + (long)qrow * q_stride + ks * 16 + 8 * g)
                     : bf16x8{};
      }
    }
    apply_qsign(qf, p.qsign);

    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // qf ready before any tile load is in flight
    int kv_end = nk;
    if (CAUSAL) kv_end = min(nk, min(q0 + rows_h, q_len));
    const int n_tiles = (kv_end + T::BC - 1) / T::BC;

    // Block-sparse: the key tiles whose 128-key block is set in either of this
    // workgroup's two 128-row mask rows, compacted in order into an LDS list
    // (FlashAttention notes (xwysyy), "Block-Sparse FlashAttention": zero
    // blocks are skipped).  Dense launches visit tiles 0 .. n_tiles-1.
    int n_iter = n_tiles;
    const uint8_t* mrow = nullptr;  // this wave's mask row
    if constexpr (SPARSE) {
      const int hm = p.mask_heads == 1 ? 0 : h;
      const uint8_t* mask0 = p.block_mask + ((long)hm * p.nbq + q0 / kSparseBlock) * p.nbk;
      const bool two_rows = q0 / kSparseBlock + 1 < p.nbq;
      // (waves whose rows lie past Nq read the last mask row; their rows are not stored)
      mrow = p.block_mask + ((long)hm * p.nbq + min(wrow0 / kSparseBlock, p.nbq - 1)) * p.nbk;
      n_iter = 0;
      for (int c0 = 0; c0 < n_tiles; c0 += kPpThreads) {
        const int j = c0 + tid;
        const int mc = j * T::BC / kSparseBlock;
        const bool vis = j < n_tiles && (mask0[mc] != 0 || (two_rows && mask0[p.nbk + mc] != 0));
        const uint64_t bal = __builtin_amdgcn_ballot_w64(vis);
        if (lane == 0) wave_count[wave] = __builtin_popcountll(bal);
        __syncthreads();
        int before = n_iter;
        for (int w = 0; w < wave; ++w) before += wave_count[w];
        const int rank = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
        if (vis) tile_list[before + rank] = j;
        for (int w = 0; w < kPpWaves; ++w) n_iter += wave_count[w];
        __syncthreads();
      }
    }
    // Key tile visited at list position t.
    auto tile_of = [&](int t) __attribute__((always_inline)) -> int {
      if constexpr (SPARSE) return tile_list[t]; else return t;
    };

    auto k_slot = [&](int c, int* row, int* colb) __attribute__((always_inline)) {
      const int rem16 = c % (16 * (DQK / 8));
      *row = 16 * (c / (16 * (DQK / 8))) + rem16 % 16;
      *colb = (rem16 / 16) * 16;
    };
    // M16: in odd 4-key groups the 16-wide d blocks are swapped pairwise, so
    // the four 16-lane blocks of a transpose read (4-key groups G, G+1, ...)
    // fall on alternate bank halves.
    auto v_slot = [&](int c, int* row, int* colb) __attribute__((always_inline)) {
      const int w = c % (DV / 2);
      const int kg = c / (DV / 2);
      *row = 4 * kg + (w % 8) / 2;
      const int blk = M16 ? (w / 8) ^ (kg & 1) : w / 8;
      *colb = (16 * blk + 8 * (w % 2)) * 2;
    };
    // Group 0 moves K tiles, group 1 V tiles; wave w of a group fills the
    // 1 KB slot runs (i*4 + w%4)*64 .. +63 of the tile (16 bytes per lane).
    // Rows past kv_end read as zero (buffer range check) and are masked.
    // (The other assignment is as correct, by the same buffer windows, and
    // measured 0.1-0.7 % slower.)
    const int gw = wave & 3;
    const bool fetch_v = grp == 1;
    const int nch = fetch_v ? CHV : CHK;  // chunks per lane of this group's tiles
    const uint32_t row_bytes = static_cast<uint32_t>(fetch_v ? v_stride : k_stride) * 2u;
    uint32_t goff[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = (i * 4 + gw) * 64 + lane;
      int row, colb;
      if (fetch_v) v_slot(c, &row, &colb); else k_slot(c, &row, &colb);
      goff[i] = row * row_bytes + colb;
    }
    const __bf16* gbase = fetch_v ? vbase : kbase;
    u32x4 stage[CH];
    // loads key tile `tile` (an index into the key sequence, not into the work list)
    auto load_tile_at = [&](int tile) __attribute__((always_inline)) {
      const int kv0 = tile * T::BC;
      const int nrows = min(kv_end - kv0, T::BC);
      const __amdgpu_buffer_rsrc_t res = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<__bf16*>(gbase + (long)kv0 * (row_bytes / 2)), (short)0, nrows * (int)row_bytes,
          kBufferFlags);
#pragma unroll
      for (int i = 0; i < CH; ++i)
        if (i < nch)
          stage[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(res, goff[i], 0, 0));
    };
    auto store_chunk = [&](__bf16* dst, auto C) __attribute__((always_inline)) {
      constexpr int i = decltype(C)::value;
      *reinterpret_cast<u32x4*>(dst + ((i * 4 + gw) * 64 + lane) * 8) = stage[i];
    };
    auto store_tile = [&](__bf16* dst) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < CH; ++i)
        if (i < nch) *reinterpret_cast<u32x4*>(dst + ((i * 4 + gw) * 64 + lane) * 8) = stage[i];
    };

    const int k_lane = M16 ? (lane >> 4) * 128 + (lane & 15) * 8
                           : ((l32 >> 4) * (DQK / 8) + g) * 128 + (l32 & 15) * 8;
    const int v_lane = M16 ? (lane >> 4) * TV::QUAD + ((lane & 15) >> 2) * 16 + 4 * (lane & 3)
                           : g * TV::QUAD + ((lane >> 4) & 1) * 64 + ((lane & 15) >> 2) * 16 + 4 * (lane & 3);
    const int v_swz = M16 ? ((lane >> 4) & 1) * 64 : 0;  // M16: odd 4-key groups' d-block swap

    const float c = p.c;
    // Tiles crossing the key tail or the diagonal (or lying wholly above this
    // wave's rows, which the mask then empties) are masked.
    // This wave's rows see the tile's 128-key block (block-sparse; else always).
    auto block_visible = [&](int tile) __attribute__((always_inline)) -> bool {
      if constexpr (SPARSE) return mrow[tile * T::BC / kSparseBlock] != 0; else return true;
    };
    auto needs_mask = [&](int tile) __attribute__((always_inline)) {
      const int kv0 = tile * T::BC;
      return (kv0 + T::BC > nk) || (CAUSAL && kv0 + T::BC - 1 > wrow0) || !block_visible(tile);
    };

    SV sv[NSV];
    u32x4 pv_op[2][2];  // P^T operands: [key block][half] (M16: [row][32-key step])
    SV acc[NACC];
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[i] = SV{};
#pragma unroll
    for (int i = 0; i < NSV; ++i) sv[i] = SV{};
    float m_run[QB], l_run[QB], m_use[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      m_run[qb] = -INFINITY;
      l_run[qb] = 0.f;
      m_use[qb] = 0.f;
    }

    // ---- MFMA phase: S_j = K_j Q^T (key blocks interleaved), then O += P_{j-1} V_{j-1}.
    // slices: one LDS operand each (M16: feeding the MFMAs of both rows)
    constexpr int kS = M16 ? 4 * KS16 : T::KT * T::KS;
    constexpr int kPv = M16 ? DB16 * 2 : T::KT * 2 * TV::DT;
    constexpr int kAhead = 3;       // LDS operand reads run this many MFMAs ahead
    constexpr int kMoveFirst = 4;   // tile-store slots inside the MFMA phase
    // 8 slices apart where that fits, else spread evenly over the phase
    constexpr int kMoveStride =
        kMoveFirst + (CH - 1) * 8 < kS + kPv ? 8 : (kS + kPv - kMoveFirst) / CH;
    static_assert(kMoveFirst + (CH - 1) * kMoveStride < kS + kPv, "move slots");
    // mid(c) runs after slice kMoveFirst + c*kMoveStride (tile chunk c moves to LDS there).
    auto mphase = [&](const __bf16* kb, const __bf16* vb, auto&& mid) __attribute__((always_inline)) {
      constexpr int n0 = kS;          // slices [0, kS): scores; [kS, kS + kPv): P V
      constexpr int nsl = kS + kPv;
      auto operand = [&](auto I) __attribute__((always_inline)) -> bf16x8 {
        constexpr int i = decltype(I)::value;
        if constexpr (M16) {
          if constexpr (i < n0) {
            constexpr int kb16 = i % 4, ks = i / 4;
            return *reinterpret_cast<const bf16x8*>(kb + k_lane + (kb16 * (DQK / 8) + 4 * ks) * 128);
          } else {
            // keys 32 k2 + 4G .. +3 and 32 k2 + 16 + 4G .. +3 of d block db
            constexpr int s = i - n0;
            constexpr int db = s % DB16, k2 = s / DB16;
            const __bf16* p0 = vb + v_lane + (db % 2 ? -v_swz : v_swz) + 8 * k2 * TV::QUAD + db * 64;
            return read_tr_pair(p0, p0 + 4 * TV::QUAD);
          }
        } else if constexpr (i < n0) {
          constexpr int kt = i % T::KT, ks = i / T::KT;
          return *reinterpret_cast<const bf16x8*>(kb + k_lane + (2 * kt * (DQK / 8) + 2 * ks) * 128);
        } else {
          constexpr int s = i - n0;
          constexpr int kt = s / (2 * TV::DT), hh = (s / TV::DT) % 2, dt = s % TV::DT;
          const __bf16* p0 = vb + v_lane + (8 * kt + 4 * hh) * TV::QUAD + dt * 128;
          return read_tr_pair(p0, p0 + 2 * TV::QUAD);
        }
      };
      bf16x8 opnd[kAhead];
      static_for<0, kAhead>([&](auto I) __attribute__((always_inline)) {
        if constexpr (decltype(I)::value < nsl) opnd[decltype(I)::value] = operand(I);
      });
      static_for<0, nsl>([&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        const bf16x8 a = opnd[i % kAhead];
        if constexpr (i + kAhead < nsl) opnd[i % kAhead] = operand(std::integral_constant<int, i + kAhead>{});
        if constexpr (M16) {
          if constexpr (i < n0) {
            constexpr int kb16 = i % 4, ks = i / 4;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              sv[kb16 * QB + qb] = mfma16(a, qf[qb * KS16 + ks], ks == 0 ? SV{} : sv[kb16 * QB + qb]);
          } else {
            constexpr int s = i - n0;
            constexpr int db = s % DB16, k2 = s / DB16;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              acc[db * QB + qb] = mfma16(a, __builtin_bit_cast(bf16x8, pv_op[qb][k2]), acc[db * QB + qb]);
          }
        } else if constexpr (i < n0) {
          constexpr int kt = i % T::KT, ks = i / T::KT;
          sv[kt] = mfma32(a, qf[ks], ks == 0 ? f32x16{} : sv[kt]);
        } else {
          constexpr int s = i - n0;
          constexpr int kt = s / (2 * TV::DT), hh = (s / TV::DT) % 2, dt = s % TV::DT;
          acc[dt] = mfma32(a, __builtin_bit_cast(bf16x8, pv_op[kt][hh]), acc[dt]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (i >= kMoveFirst && (i - kMoveFirst) % kMoveStride == 0 &&
                      (i - kMoveFirst) / kMoveStride < CH) {
          mid(std::integral_constant<int, (i - kMoveFirst) / kMoveStride>{});
          __builtin_amdgcn_sched_barrier(0);
        }
      });
    };
    // A key is visible to row qb of this lane when it lies below key_lim[qb]
    // (and its block is set, block-sparse).  Every score position of a lane is
    // a compile-time offset from the lane's first key, so the mask is one
    // compare per score against t = key_lim - kv0 - (lane's first key).
    int key_lim[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) key_lim[qb] = CAUSAL ? min(nk, qrow_of(qb) + 1) : nk;
    auto apply_mask = [&](int tile) __attribute__((always_inline)) {
      const int kv0 = tile * T::BC;
      const bool bvis = block_visible(tile);
      if constexpr (M16) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int t = bvis ? key_lim[qb] - kv0 - 4 * (lane >> 4) : -1;
#pragma unroll
          for (int kb16 = 0; kb16 < 4; ++kb16)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (!(16 * kb16 + r < t)) sv[kb16 * QB + qb][r] = -INFINITY;
        }
      } else {
        const int t = bvis ? key_lim[0] - kv0 - 4 * g : -1;
#pragma unroll
        for (int kt = 0; kt < T::KT; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (!(kt * 32 + 8 * (r >> 2) + (r & 3) < t)) sv[kt][r] = -INFINITY;
      }
    };
    // ---- VALU phase: online softmax of S_j -> P_j, O rescale when the max moved.
    // Exponentials of the tile against the running max, packed to bf16 into
    // pv_op; returns this lane's partial row sum in ls0 + ls1.
    // this lane's partial row sums: ls[qb][0] + ls[qb][1] for row qb
    auto exps = [&](float (&ls)[QB][2]) __attribute__((always_inline)) {
      auto expo = [](int e, float x) __attribute__((always_inline)) {
        return (e % 8) < kExp2Poly / 4 ? exp2_poly(x) : __builtin_amdgcn_exp2f(x);
      };
      if constexpr (M16) {
        // P^T operand of 32-key step k2, row qb: keys 4G..4G+3 of key block
        // 2 k2, then the same of key block 2 k2 + 1
#pragma unroll
        for (int kb16 = 0; kb16 < 4; ++kb16)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
              const float e0 = expo(4 * kb16 + r, fmaf(sv[kb16 * QB + qb][r], c, -m_use[qb]));
              const float e1 = expo(4 * kb16 + r + 1, fmaf(sv[kb16 * QB + qb][r + 1], c, -m_use[qb]));
              if (kb16 == 0 && r == 0) {
                ls[qb][0] = e0;
                ls[qb][1] = e1;
              } else {
                ls[qb][0] += e0;
                ls[qb][1] += e1;
              }
              const bf16x2 pk = {(__bf16)e0, (__bf16)e1};
              uint32_t u = __builtin_bit_cast(uint32_t, pk);
              asm volatile("" : "+v"(u));  // convert here, not among the next phase's MFMAs
              pv_op[qb][kb16 / 2][(kb16 % 2) * 2 + r / 2] = u;
            }
      } else {
#pragma unroll
        for (int kt = 0; kt < T::KT; ++kt)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float e0 = expo(16 * kt + r, fmaf(sv[kt][r], c, -m_use[0]));
            const float e1 = expo(16 * kt + r + 1, fmaf(sv[kt][r + 1], c, -m_use[0]));
            if (kt == 0 && r == 0) {
              ls[0][0] = e0;
              ls[0][1] = e1;
            } else {
              ls[0][0] += e0;
              ls[0][1] += e1;
            }
            const bf16x2 pk = {(__bf16)e0, (__bf16)e1};
            uint32_t u = __builtin_bit_cast(uint32_t, pk);
            asm volatile("" : "+v"(u));  // convert here, not among the next phase's MFMAs
            pv_op[kt][r >> 3][(r & 7) >> 1] = u;
          }
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        asm volatile("" : "+v"(ls[qb][0]), "+v"(ls[qb][1]));  // keep the sums in this phase
    };
    // any row of the lane without a running max yet
    auto no_max_yet = [&]() __attribute__((always_inline)) {
      bool r = m_run[0] == -INFINITY;
      if constexpr (QB > 1) r = r || m_run[1] == -INFINITY;
      return r;
    };
    auto vphase = [&](int j) __attribute__((always_inline)) {
      const int tile = tile_of(j);
      if (needs_mask(tile)) apply_mask(tile);
      float ls[QB][2];
      // Once every row of the wave has a running max, the exponentials are
      // taken against it first.  A lane's partial sum bounds each of its
      // exponentials, so when no lane's sum exceeds 2^tau no score of the
      // tile exceeds its row's max by more than tau: the rescale would not
      // fire and the tile is done without its row maxima.  Otherwise the
      // exact step below runs (and decides as before), so the results are
      // bitwise those of that step alone.
      bool done = false;
      if (__builtin_amdgcn_ballot_w64(no_max_yet()) == 0) {
        exps(ls);
        bool big = ls[0][0] + ls[0][1] > kTwoPowTau;
        if constexpr (QB > 1) big = big || ls[1][0] + ls[1][1] > kTwoPowTau;
        done = __builtin_amdgcn_ballot_w64(big) == 0;
      }
      if (!done) {
        float mx[QB];
        if constexpr (M16) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
            for (int kb16 = 0; kb16 < 4; kb16 += 2) {
              m0 = max3f(m0, sv[kb16 * QB + qb][0], sv[kb16 * QB + qb][1]);
              m0 = max3f(m0, sv[kb16 * QB + qb][2], sv[kb16 * QB + qb][3]);
              m1 = max3f(m1, sv[(kb16 + 1) * QB + qb][0], sv[(kb16 + 1) * QB + qb][1]);
              m1 = max3f(m1, sv[(kb16 + 1) * QB + qb][2], sv[(kb16 + 1) * QB + qb][3]);
            }
            mx[qb] = pair_max(pair16_max(max3f(m0, m1, -INFINITY))) * c;
          }
        } else {
          float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
          for (int e = 0; e < 32; e += 4) {
            m0 = max3f(m0, sv[e / 16][e % 16], sv[e / 16][e % 16 + 1]);
            m1 = max3f(m1, sv[e / 16][e % 16 + 2], sv[e / 16][e % 16 + 3]);
          }
          mx[0] = pair_max(max3f(m0, m1, -INFINITY)) * c;
        }
        // The rescale (new max, alpha, l and O scaled) runs only when some
        // row's max grew by more than tau; the test is wave-uniform, and
        // otherwise alpha would be exactly 1.
        bool grow = mx[0] > m_run[0] + kTau;
        if constexpr (QB > 1) grow = grow || mx[1] > m_run[1] + kTau;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const float m_new = fmaxf(m_run[qb], mx[qb]);
            const float alpha =
                (m_run[qb] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
            m_run[qb] = m_new;
            m_use[qb] = (m_new == -INFINITY) ? 0.f : m_new;
            l_run[qb] *= alpha;
            if constexpr (M16) {
#pragma unroll
              for (int db = 0; db < DB16; ++db) acc[db * QB + qb] *= alpha;
            } else {
#pragma unroll
              for (int dt = 0; dt < TV::DT; ++dt) acc[dt] *= alpha;
            }
          }
        }
        exps(ls);
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) l_run[qb] += ls[qb][0] + ls[qb][1];
    };

    // ---- schedule.  Half periods h = 0, 1, ...: group 0 runs M_j at h = 2j and
    // V_j at h = 2j+1, group 1 runs M_j at h = 2j+1 and V_j at h = 2j+2.  K_t
    // lives in k[t%2], V_t in v[t%2].  Tiles move global -> VGPRs -> LDS:
    // during M_j, between two MFMAs, the V mover (group 1) stores V_j (loaded
    // one period earlier) and the K mover (group 0) stores K_{j+1}; at the
    // start of V_j (block-sparse: at the end of M_j) they load V_{j+1} and
    // K_{j+2}.  Each store is complete before the barrier that ends its phase,
    // which precedes the first read of the tile.  V_j is written in v[j%2]
    // during M_j of either group (V_{j-2} there was last read in M_{j-1}) and
    // first read in M_{j+1}; K_{j+1} in k[(j+1)%2] likewise (K_{j-1} last read
    // in M_{j-1}, K_{j+1} first read in M_{j+1}).
    constexpr bool kLoadInMfmaPhase = SPARSE;
    auto kbuf = [&](auto I) __attribute__((always_inline)) -> __bf16* {
      if constexpr (decltype(I)::value % 2 == 0) return k_lds0; else return k_lds1;
    };
    auto vbuf = [&](auto I) __attribute__((always_inline)) -> __bf16* {
      if constexpr (decltype(I)::value % 2 == 0) return v_lds0; else return v_lds1;
    };
    auto barrier = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kForceSafe) __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    // One period: M_j (+ tile store and load), barrier, V_j, barrier.  At j = 0
    // the P V adds zero (P and the V buffer it reads are zeroed first); at
    // j = n_iter the scores come from a stale K tile and are never used.
    auto period = [&](int j, auto J) __attribute__((always_inline)) {
      constexpr int j2 = decltype(J)::value;  // j % 2
      const int st = fetch_v ? j : j + 1;  // tile stored in this phase
      // the tile loaded at the start of the VALU phase; looked up now, so that a
      // work-list read (block-sparse) is done by then
      const int next_tile = st + 1 < n_iter ? tile_of(st + 1) : 0;
      __bf16* dst = fetch_v ? vbuf(std::integral_constant<int, j2>{}) : kbuf(std::integral_constant<int, j2 + 1>{});
      // The staged tile goes to LDS one 16-byte chunk per lane at a time,
      // spread over the MFMA phase; the next tile is loaded into the freed
      // registers at the start of the VALU phase, which is the shorter one
      // (dense), or right after the last chunk (block-sparse, whose VALU phase
      // masks more tiles: there the MFMA-phase placement measured faster).
      // Past the last tile the store is left unguarded: it writes stale
      // registers into a buffer no later MFMA phase reads.
      auto move = [&](auto C) __attribute__((always_inline)) {
        constexpr int c = decltype(C)::value;
        if (c < nch) store_chunk(dst, C);
        if constexpr (kForceSafe) barrier();
        if constexpr (kLoadInMfmaPhase && c == CH - 1) {
          if (st + 1 < n_iter) load_tile_at(next_tile);
        }
      };
      // The wave in its MFMA phase gets issue priority over the other wave of
      // its SIMD, so a ready MFMA is not held behind that wave's softmax.
      __builtin_amdgcn_s_setprio(3);
      mphase(kbuf(std::integral_constant<int, j2>{}), vbuf(std::integral_constant<int, j2 + 1>{}), move);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // this phase's LDS stores are done
      barrier();
      if constexpr (!kLoadInMfmaPhase) {
        if (st + 1 < n_iter) load_tile_at(next_tile);
      }
      if (j < n_iter) vphase(j);
      barrier();
    };

#pragma unroll
    for (int kt = 0; kt < T::KT; ++kt) pv_op[kt][0] = pv_op[kt][1] = u32x4{};
    for (int i = tid; i < TV::V_ELEMS / 8; i += kPpThreads)
      reinterpret_cast<u32x4*>(v_lds1)[i] = u32x4{};
    // prologue: K_0 stored and K_1 loaded (K mover); V_0 loaded (V mover)
    if (fetch_v) {
      if (n_iter > 0) load_tile_at(tile_of(0));
    } else {
      if (n_iter > 0) { load_tile_at(tile_of(0)); __builtin_amdgcn_s_waitcnt(kWaitVm0); store_tile(k_lds0); }
      if (n_iter > 1) load_tile_at(tile_of(1));
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    barrier();
    if (!kForceSafe && grp == 1) barrier();  // group 1 starts half a period late
    int j = 0;
    for (; j + 1 <= n_iter; j += 2) {
      period(j, std::integral_constant<int, 0>{});
      period(j + 1, std::integral_constant<int, 1>{});
    }
    if (j <= n_iter) period(j, std::integral_constant<int, 0>{});
    if (!kForceSafe && grp == 0) barrier();

    float l_tot[QB], inv[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      l_tot[qb] = M16 ? pair_sum(pair16_sum(l_run[qb])) : pair_sum(l_run[qb]);
      inv[qb] = l_tot[qb] > 0.f ? 1.f / l_tot[qb] : 0.f;
    }
    // O leaves through LDS.  A lane's accumulator holds 4-column pieces of one
    // row, so storing it directly scatters every store instruction over 32
    // rows.  Instead each wave writes its 32 x DV block, normalised, in bf16,
    // row-major into 8 KB of the K/V buffers (after the last barrier no wave
    // reads them), then stores whole rows with 16-byte stores.  The 16-byte
    // chunks of row r sit at chunk index XOR (r % 16), so that neither the
    // column-wise writes nor the row-wise reads conflict on LDS banks.
    __bf16* const ost = (wave < 2 ? k_lds0 : wave < 4 ? k_lds1 : wave < 6 ? v_lds0 : v_lds1) +
                        (wave & 1) * (kRowsPerWave * DV);
    if constexpr (M16) {
      // lane l: row 16 qb + l%16, columns 16 db + 4 (l/16) .. +3
#pragma unroll
      for (int db = 0; db < DB16; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          bf16x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(acc[db * QB + qb][e] * inv[qb]);
          const int r = 16 * qb + (lane & 15);
          const int chk = (2 * db + (lane >> 5)) ^ (r % kOChunks);
          *reinterpret_cast<bf16x4*>(ost + r * DV + chk * 8 + 4 * ((lane >> 4) & 1)) = ov;
        }
    } else {
#pragma unroll
      for (int dt = 0; dt < TV::DT; ++dt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          bf16x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(acc[dt][4 * rq + e] * inv[0]);
          const int chk = (dt * 4 + rq) ^ (l32 % kOChunks);  // columns dt*32 + 8 rq .. +7
          *reinterpret_cast<bf16x4*>(ost + l32 * DV + chk * 8 + 4 * g) = ov;
        }
    }
    // the wave's LDS writes precede its reads of other lanes' data
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    __bf16* const obase = p.o + (q_row0 + wrow0) * o_stride + (long)h * DV;
    constexpr int kRowsPerPass = 64 / kOChunks;
    const int cc = lane % kOChunks;
#pragma unroll
    for (int i = 0; i < kRowsPerWave / kRowsPerPass; ++i) {
      const int r = i * kRowsPerPass + lane / kOChunks;
      const u32x4 ov = *reinterpret_cast<const u32x4*>(ost + r * DV + (cc ^ (r % kOChunks)) * 8);
      if (wrow0 + r < q_len) *reinterpret_cast<u32x4*>(obase + r * o_stride + cc * 8) = ov;
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qr = qrow_of(qb);
      if (qr < q_len && (M16 ? (lane >> 4) == 0 : g == 0))
        p.lse[lse_base + (long)h * lse_hstride + qr] =
            l_tot[qb] > 0.f ? (m_run[qb] + log2f(l_tot[qb])) * kLn2 : -INFINITY;
    }
  };

  // Paired items: workgroup w of XCD x (w = x + 8 m) runs, within that XCD's
  // items x + 8 r (decode_work), the i-th and the (n-1-i)-th item of one unit
  // of n items, so a pair costs about the same under the causal mask (items
  // run longest first) and the hardware still balances pairs between CUs.
  // One launch gap and one pipeline fill less per pair.  Otherwise each
  // workgroup runs the item of its own id.
  if (p.paired) {
    const int n = p.nqb * (p.G / p.pack);  // items per unit
    const int xcd = blockIdx.x % kXcds, m = blockIdx.x / kXcds;
    const int u = m / (n / 2), i = m % (n / 2);
    run_item((u * n + i) * kXcds + xcd);
    __syncthreads();  // the first item's LDS reads are done before the second's stores
    run_item((u * n + n - 1 - i) * kXcds + xcd);
  } else {
    run_item(blockIdx.x);
  }
}

// ---------------------------------------------------------------------------
// LPT order of the sequences of a packed batch (FlashAttention-4 (papercache
// summary), section 3.3): a counting sort, in one workgroup, of the sequences
// by the key-tile count of their longest work tile, longest first.
constexpr int kPlanThreads = 1024;
constexpr int kPlanBuckets = 8192;          // keys >= kPlanBuckets - 1 share the top bucket
constexpr int kPlanPer = kPlanBuckets / kPlanThreads;

__global__ __launch_bounds__(kPlanThreads) void varlen_plan_kernel(const int32_t* cu_q,
                                                                    const int32_t* cu_k, int n,
                                                                    int max_q, int max_k,
                                                                    int causal, int32_t* order) {
  __shared__ int hist[kPlanBuckets];
  __shared__ int part[kPlanThreads];
  const int tid = threadIdx.x;
  for (int i = tid; i < kPlanBuckets; i += kPlanThreads) hist[i] = 0;
  __syncthreads();
  auto key = [&](int z) {
    const int lq = min(max(cu_q[z + 1] - cu_q[z], 0), max_q);
    const int lk = min(max(cu_k[z + 1] - cu_k[z], 0), max_k);
    const int w = causal ? min(lq, lk) : lk;
    return min((w + 63) / 64, kPlanBuckets - 1);
  };
  for (int z = tid; z < n; z += kPlanThreads) atomicAdd(&hist[key(z)], 1);
  __syncthreads();
  // Exclusive scan in descending key order: thread t owns the kPlanPer
  // buckets counted from the top, (kPlanBuckets-1 - t*kPlanPer) downwards.
  int sum = 0;
  for (int i = 0; i < kPlanPer; ++i) sum += hist[kPlanBuckets - 1 - (tid * kPlanPer + i)];
  part[tid] = sum;
  __syncthreads();
  for (int step = 1; step < kPlanThreads; step *= 2) {
    const int add = tid >= step ? part[tid - step] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  int run = part[tid] - sum;  // buckets of higher key than this thread's first
  for (int i = 0; i < kPlanPer; ++i) {
    const int kb = kPlanBuckets - 1 - (tid * kPlanPer + i);
    const int c = hist[kb];
    hist[kb] = run;  // becomes the next free position of bucket kb
    run += c;
  }
  __syncthreads();
  for (int z = tid; z < n; z += kPlanThreads) order[atomicAdd(&hist[key(z)], 1)] = z;
}


constexpr bool use_pp(int d) { return d == 128; }

// Query heads of one KV group that a ping-pong workgroup takes together (its
// 256 rows are 256 / pack rows of each): the largest power of two up to 8
// dividing the group size.  Under the causal mask, a workgroup's rows then
// span fewer keys, so fewer tiles cross the diagonal; the K/V tile still
// serves 256 rows.
constexpr int pp_pack(int G) { return G % 8 == 0 ? 8 : G % 4 == 0 ? 4 : G % 2 == 0 ? 2 : 1; }

// Ping-pong launches pair the items of a unit when a unit has an even count
// and keys number at most kPairMaxKeys; not block-sparse ones, whose item
// costs follow the mask rather than the diagonal (pairing measured 2 % slower
// there).  Longer sequences gain nothing from pairs (an item's launch gap is
// a small share of it) and lose L2 reuse: a pair's short item streams the
// start of the key range while the XCD's other workgroups are further on
// (N = 32768: 8.1 instead of 4.7 GB of HBM traffic).  Returns the workgroups
// to launch and sets p.items and p.paired.
constexpr int kPairMaxKeys = 8192;

int pp_grid(Params& p, long items, bool pair) {
  p.items = static_cast<int>(items);
  const int n = p.nqb * (p.G / p.pack);
  p.paired = (pair && p.Nk <= kPairMaxKeys && n % 2 == 0) ? 1 : 0;
  return static_cast<int>(p.paired ? items / 2 : items);
}

template <int D, bool CAUSAL, bool VARLEN>
int launch_one(Params p, int grid, hipStream_t stream) {
  (void)hipGetLastError();  // clear a stale error so the check below is ours
  p.items = grid;
  p.paired = 0;
  if constexpr (use_pp(D)) {
    const int wgs = pp_grid(p, grid, true);
    hipLaunchKernelGGL((attn_fwd_pp_kernel<D, D, CAUSAL, VARLEN, false, kPpMfma16>), dim3(wgs),
                       dim3(kPpThreads), 0, stream, p);
  }
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, VARLEN>), dim3(grid), dim3(kThreads), 0, stream,
                       p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    attn_detail::last_hip_error = static_cast<int>(e);
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

// Work items for `units` (batch, KV head) units of `per_unit` items each,
// units padded to a multiple of the XCD count (decode_work); a ping-pong
// launch runs two items per workgroup (pp_grid).
long grid_size(long units, long per_unit) { return (units + kXcds - 1) / kXcds * kXcds * per_unit; }

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

int check_common(int Hq, int Hkv, int d, float scale) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_HEADS;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (!std::isfinite(scale)) return ATTN_ERR_SIZE;
  return ATTN_OK;
}

// Scale into the kernel's form: c = |scale| * log2(e) and the sign, which the
// kernels fold into the query fragments (apply_qsign).
void set_scale(Params& p, float scale) {
  const double a = std::fabs(static_cast<double>(scale));
  p.c = static_cast<float>((scale == 0.f ? 1.0 : a) * 1.4426950408889634);
  p.qsign = scale > 0.f ? 1 : scale < 0.f ? -1 : 0;
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
  const int pack = use_pp(d) ? pp_pack(Hq / Hkv) : 1;
  const int br = use_pp(d) ? kPpBr / pack : kBr;
  const long nqb = (Nq + br - 1) / br;
  const long grid = grid_size((long)B * Hkv, (long)nqb * (Hq / Hkv / pack));
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
  p.pack = pack;
  p.num_seqs = B;
  set_scale(p, scale);
  return dispatch(p, d, causal != 0, false, static_cast<int>(grid),
                  static_cast<hipStream_t>(stream));
}

extern "C" int attn_fwd_dims(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int Hq, int Hkv, int Nq, int Nk, int d_qk, int d_v, float scale,
                             int causal, const int32_t* seqlens_k, void* stream) {
  if (d_qk == d_v)
    return attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d_qk, scale, causal, seqlens_k, stream);
  if (B < 0 || Nq < 0 || Nk < 0) return ATTN_ERR_SIZE;
  int rc = check_common(Hq, Hkv, 128, scale);
  if (rc != ATTN_OK) return rc;
  if (!(d_qk == 192 && d_v == 128)) return ATTN_ERR_HEAD_DIM;
  if (B == 0 || Nq == 0) return ATTN_OK;
  rc = check_buffers(q, k, v, o, lse, Nk > 0);
  if (rc != ATTN_OK) return rc;
  const int pack = pp_pack(Hq / Hkv);
  const long nqb = (Nq + kPpBr / pack - 1) / (kPpBr / pack);
  const long grid = grid_size((long)B * Hkv, (long)nqb * (Hq / Hkv / pack));
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
  p.pack = pack;
  p.num_seqs = B;
  set_scale(p, scale);
  const unsigned wgs = static_cast<unsigned>(pp_grid(p, grid, true));
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (causal)
    hipLaunchKernelGGL((attn_fwd_pp_kernel<192, 128, true, false>), dim3(wgs), dim3(kPpThreads), 0,
                       st, p);
  else
    hipLaunchKernelGGL((attn_fwd_pp_kernel<192, 128, false, false>), dim3(wgs), dim3(kPpThreads), 0,
                       st, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    attn_detail::last_hip_error = static_cast<int>(e);
    return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

extern "C" int attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o,
                                    float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                    float scale, int causal, const int32_t* seqlens_k,
                                    const uint8_t* block_mask, int mask_heads, void* stream) {
  if (B < 0 || Nq < 0 || Nk < 0) return ATTN_ERR_SIZE;
  int rc = check_common(Hq, Hkv, d, scale);
  if (rc != ATTN_OK) return rc;
  if (d != 128) return ATTN_ERR_HEAD_DIM;
  if (mask_heads != 1 && mask_heads != Hq) return ATTN_ERR_HEADS;
  if (B == 0 || Nq == 0) return ATTN_OK;
  if (block_mask == nullptr) return ATTN_ERR_NULL;
  rc = check_buffers(q, k, v, o, lse, Nk > 0);
  if (rc != ATTN_OK) return rc;
  if ((long)Nk > (long)kMaxSparseTiles * 64) return ATTN_ERR_TOO_LARGE;
  const long nqb = (Nq + kPpBr - 1) / kPpBr;
  const long grid = grid_size((long)B * Hkv, (long)nqb * (Hq / Hkv));
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
  p.pack = 1;  // the mask is per 128-row block of one head
  p.num_seqs = B;
  set_scale(p, scale);
  p.block_mask = block_mask;
  p.mask_heads = mask_heads;
  p.nbq = (Nq + kSparseBlock - 1) / kSparseBlock;
  p.nbk = (Nk + kSparseBlock - 1) / kSparseBlock;
  const unsigned wgs = static_cast<unsigned>(pp_grid(p, grid, false));
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (causal)
    hipLaunchKernelGGL((attn_fwd_pp_kernel<128, 128, true, false, true, kPpMfma16>), dim3(wgs),
                       dim3(kPpThreads), 0, st, p);
  else
    hipLaunchKernelGGL((attn_fwd_pp_kernel<128, 128, false, false, true, kPpMfma16>), dim3(wgs),
                       dim3(kPpThreads), 0, st, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    attn_detail::last_hip_error = static_cast<int>(e);
    return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

extern "C" int attn_fwd_varlen_ordered(const void* q, const void* k, const void* v, void* o,
                                       float* lse, const int32_t* cu_seqlens_q,
                                       const int32_t* cu_seqlens_k, int num_seqs, int Hq, int Hkv,
                                       int max_seqlen_q, int max_seqlen_k, int d, float scale,
                                       int causal, const int32_t* seq_order, void* stream) {
  if (num_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return ATTN_ERR_SIZE;
  int rc = check_common(Hq, Hkv, d, scale);
  if (rc != ATTN_OK) return rc;
  if (num_seqs == 0 || max_seqlen_q == 0) return ATTN_OK;
  if (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr) return ATTN_ERR_NULL;
  rc = check_buffers(q, k, v, o, lse, max_seqlen_k > 0);
  if (rc != ATTN_OK) return rc;
  const int pack = use_pp(d) ? pp_pack(Hq / Hkv) : 1;
  const int br = use_pp(d) ? kPpBr / pack : kBr;
  const long nqb = (max_seqlen_q + br - 1) / br;
  const long grid = grid_size((long)num_seqs * Hkv, (long)nqb * (Hq / Hkv / pack));
  if (grid > INT_MAX) return ATTN_ERR_TOO_LARGE;
  Params p{};
  p.q = static_cast<const __bf16*>(q);
  p.k = static_cast<const __bf16*>(k);
  p.v = static_cast<const __bf16*>(v);
  p.o = static_cast<__bf16*>(o);
  p.lse = lse;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.seq_order = seq_order;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.Nq = max_seqlen_q;
  p.Nk = max_seqlen_k;
  p.nqb = static_cast<int>(nqb);
  p.pack = pack;
  p.num_seqs = num_seqs;
  set_scale(p, scale);
  return dispatch(p, d, causal != 0, true, static_cast<int>(grid),
                  static_cast<hipStream_t>(stream));
}

extern "C" int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int num_seqs, int Hq, int Hkv, int max_seqlen_q, int max_seqlen_k,
                               int d, float scale, int causal, void* stream) {
  return attn_fwd_varlen_ordered(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, num_seqs, Hq, Hkv,
                                 max_seqlen_q, max_seqlen_k, d, scale, causal, nullptr, stream);
}

extern "C" int attn_varlen_plan(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int num_seqs, int max_seqlen_q, int max_seqlen_k, int causal,
                                int32_t* seq_order, void* stream) {
  if (num_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return ATTN_ERR_SIZE;
  if (num_seqs == 0) return ATTN_OK;
  if (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr || seq_order == nullptr)
    return ATTN_ERR_NULL;
  (void)hipGetLastError();
  hipLaunchKernelGGL(varlen_plan_kernel, dim3(1), dim3(kPlanThreads), 0,
                     static_cast<hipStream_t>(stream), cu_seqlens_q, cu_seqlens_k, num_seqs,
                     max_seqlen_q, max_seqlen_k, causal != 0 ? 1 : 0, seq_order);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    attn_detail::last_hip_error = static_cast<int>(e);
    return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

extern "C" const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_HEAD_DIM: return "unsupported head dimension (supported: 64, 128)";
    case ATTN_ERR_HEADS: return "bad head counts (need Hq >= 1, Hkv >= 1, Hq % Hkv == 0)";
    case ATTN_ERR_SIZE: return "negative size, or scale not finite";
    case ATTN_ERR_LAUNCH: return "HIP kernel launch failed (see attn_last_hip_error)";
    case ATTN_ERR_ALIGN: return "q/k/v/o must be 16-byte aligned and lse 4-byte aligned";
    case ATTN_ERR_TOO_LARGE: return "problem too large for 32-bit grid or row indexing";
    case ATTN_ERR_SCRATCH:
      return "B * Hq * Nq exceeds the 4194304 rows of attn_bwd_noalloc's static scratch";
    default: return "unknown attn status";
  }
}

extern "C" int attn_last_hip_error(void) { return attn_detail::last_hip_error; }

extern "C" const char* attn_version(void) { return "0.1.0"; }
