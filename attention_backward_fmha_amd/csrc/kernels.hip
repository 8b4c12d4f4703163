// kernels.hip -- the three device stages of the attention backward on gfx950 (CDNA4).
//
// Stage 1 (k_dot):     D[h][row] = sum_c dO[row,h,c] * O[row,h,c] and LSE*log2(e)  HBM bound
// Stage 2 (k_bwd_main): one work item per (segment b, K/V head g, key tile j):
//     for every query head h of g's group and every query block i the mask lets tile j see:
//       S = Q_i K_j^T, P = exp(scale*S - LSE_i) (0 where masked), dP = dO_i V_j^T,
//       dS = P * (dP - D_i), dV_j += P^T dO_i, dK_j += dS^T Q_i, dQ_i += dS K_j
//     dK_j (scaled) and dV_j are written once at the end; the tile's dS K_j goes to the dQ
//     accumulator: the item's split (deterministic), an fp32 atomic add into the one split,
//     or a packed bf16 atomic add into the segment's bf16 slot.                     MFMA bound
// Stage 3 (k_dq_reduce): dQ = bf16(scale * sum_{splits that wrote the block} acc), the fp32
//     sum in ascending split order (one split, fp32 or bf16, in the atomic modes).  HBM bound
//
// Matrix products use v_mfma_f32_32x32x16_bf16 (bf16 operands, fp32 accumulation).  Its lane
// layout (checked on the device): lane l holds row (l % 32) of A and column (l % 32) of B with
// the 8 reduction-index values 8*(l/32) .. 8*(l/32)+7; result element (i, j) sits in lane
// j + 32*((i/4)%2), register 4*(i/8) + i%4.  A sum over the reduction index does not depend on
// the order of its terms, so any assignment of reduction indices to (lane half, slot) works as
// long as A and B use the same one; the kernels use that to feed P and dS straight from the
// result registers of S and dP into the next products.
//
// The K operand of dQ (reduction over keys, which run along the K tile's rows) is read once
// per work item with ds_read_b64_tr_b16: in each 16-lane group, lane s points at 4 consecutive
// elements of row (s/4), columns 4*(s%4)..4*(s%4)+3 of a 4x16 block, and lane i receives
// column i of the block (4 values, one per row).
#include "device.h"
#include "kernels.h"
#include "tiling.h"

namespace fmha {
namespace {

// ------------------------------------------------------------------------------------------
// Stage 1: D = rowsum(dO * O).  DV/8 lanes per row, 16 bytes per lane per tensor.
// ------------------------------------------------------------------------------------------
// Steps of work group w of the wide kernel (grid order; group mode, 32-row blocks, 256-key
// tiles): the (query head, query block) pairs of its item's tiles, shared evenly by the
// item's parts, plus a constant for the tile loads and the epilogue; 0 for a work group
// whose segment has no such tile.
__device__ int wide_steps(const KParams& p, const int* seqstart_q, const int* seqstart_k, int w) {
  const int nbh = p.Hkv * p.B;
  const int ip = w / nbh;
  const int item = ip / p.kv_parts;
  const int part = ip - item * p.kv_parts;
  const int b = (w - ip * nbh) / p.Hkv;
  const int lq = seqstart_q[b + 1] - seqstart_q[b];
  const int lk = seqstart_k[b + 1] - seqstart_k[b];
  const MaskGeom mg = mask_geom(p.mask_type, p.window_left, p.window_right, lq, lk);
  int steps = 0;
  for (int tsub = 0; tsub < p.tiles_per_item; ++tsub) {
    const int j = item * p.tiles_per_item + tsub;
    if (j * 256 >= lk) break;
    int64_t lo, hi;
    rows_for_keys(mg, lq, (int64_t)j * 256, min(j * 256 + 255, lk - 1), &lo, &hi);
    if (hi >= lo) steps += ((int)hi / 32 - (int)lo / 32 + 1) * p.group_size;
  }
  if (steps == 0) return 0;
  return steps * (part + 1) / p.kv_parts - steps * part / p.kv_parts + 6;
}

constexpr int kOrderSegs = 1025;  // segment offsets staged in LDS for up to 1024 segments

// The wide kernel's work groups (at most 2048) sorted by the key
// (65535 - steps) * 2048 + w, i.e. most steps first and ties in grid order, with a bitonic
// network in LDS; order[i] is the work group of rank i.  Run by the first work group of the D
// stage, so it costs no launch of its own and overlaps that stage's memory traffic.
__device__ void order_work_groups(const KParams& p, int* key, int* seg) {
  const int n = p.order_n;
  int N = 2;
  while (N < n) N <<= 1;
  // the segment offsets come to LDS in one round of loads, not eight dependent ones per
  // thread that would wait behind the stage's HBM stream
  const int* sq = p.seqstart_q;
  const int* sk = p.seqstart_k;
  if (p.B < kOrderSegs) {
    for (int i = threadIdx.x; i <= p.B; i += blockDim.x) {
      seg[i] = sq[i];
      seg[kOrderSegs + i] = sk[i];
    }
    __syncthreads();
    sq = seg;
    sk = seg + kOrderSegs;
  }
  for (int w = threadIdx.x; w < N; w += blockDim.x)
    key[w] = w < n ? ((65535 - min(wide_steps(p, sq, sk, w), 65535)) << 11) | w : 0x7fffffff;
  __syncthreads();
  // 256 threads, at most 1024 pairs per stage: the loads of a thread's four pairs are issued
  // before any comparison, so a stage costs one LDS round trip rather than four
  constexpr int PT = 4;
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      int a[PT], c[PT];
#pragma unroll
      for (int u = 0; u < PT; ++u) {
        const int t = threadIdx.x + 256 * u;
        const int i = 2 * t - (t & (j - 1));  // 2j * (t / j) + t % j, j a power of two
        if (t < N / 2) {
          a[u] = key[i];
          c[u] = key[i + j];
        }
      }
#pragma unroll
      for (int u = 0; u < PT; ++u) {
        const int t = threadIdx.x + 256 * u;
        const int i = 2 * t - (t & (j - 1));
        if (t < N / 2 && (a[u] > c[u]) == ((i & k) == 0)) {
          key[i] = c[u];
          key[i + j] = a[u];
        }
      }
      __syncthreads();
    }
  }
  for (int r = threadIdx.x; r < n; r += blockDim.x) p.order[r] = key[r] & 2047;
}

constexpr int kDotRows = 64;  // rows of one query head per work group of k_dot

template <int DV>
__global__ __launch_bounds__(256) void k_dot(const KParams p) {
  // with a cost order, work group 0 builds it (dispatched first, it overlaps the others)
  const int blk = (int)blockIdx.x - (p.order_n > 0 ? 1 : 0);
  if (blk < 0) {
    __shared__ int key[2048];
    __shared__ int seg[2 * kOrderSegs];
    order_work_groups(p, key, seg);
    return;
  }
  // Work group = 64 consecutive rows of one query head, so the LSE reads and the D / scaled-LSE
  // writes are contiguous runs; LPR lanes share a row, each pass covers RPP rows, and the
  // loads of all passes are issued before the products.
  constexpr int LPR = DV / 8;
  constexpr int RPP = 256 / LPR;
  constexpr int NP = kDotRows / RPP;
  const int tid = threadIdx.x;
  const int c8 = tid % LPR;
  const int h = blk % p.Hq;
  const int64_t row0 = (int64_t)(blk / p.Hq) * kDotRows + tid / LPR;
  const bool group = p.seqstart_q != nullptr;
  bf16x8 a[NP], o[NP];
  int bs[NP];
  int64_t trs[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int64_t row = row0 + j * RPP;
    int b = 0;
    int64_t trow = row;
    if (!group) {
      b = (int)(row / p.Sq);
      trow = row - (int64_t)b * p.Sq;
    }
    bs[j] = b;
    trs[j] = trow;
    if (row < p.rows_q) {
      a[j] = *(const bf16x8*)(p.dout + elem_off(p.do_s, group, b, trow, h) + c8 * 8);
      o[j] = *(const bf16x8*)(p.o + elem_off(p.o_s, group, b, trow, h) + c8 * 8);
    }
  }
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int64_t row = row0 + j * RPP;
    const bool valid = row < p.rows_q;
    float acc = 0.f;
    if (valid) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += (float)a[j][e] * (float)o[j][e];
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
    if (valid && c8 == 0) {
      const float l2 = p.lse[(group ? 0 : (int64_t)bs[j] * p.lse_s[0]) + (int64_t)h * p.lse_s[1] + trs[j]] * kLog2e;
      p.dsum[(int64_t)h * p.rows_q + row] = acc;
      p.lse2[(int64_t)h * p.rows_q + row] = l2;
    }
  }
}

// ------------------------------------------------------------------------------------------
// Stage 2: the main kernel.  256 threads = 4 waves; wave w owns 32 keys of the tile (keys
// 32w .. 32w+31, spread over its lanes by kmap below).
//
// The (query head, query block) steps of a work item form one flat loop.  While step n is
// computed, the global loads of step n+1 are in flight into registers; after the step's second
// barrier they are written to LDS twice: row-major (the A operand of S and dP) and transposed
// with the block's queries along the row (the B operand of dV and dK).  The transposed copies
// store queries in the order the P/dS result registers feed the reduction slots, so every
// operand of S, dP, dV and dK is a plain 16-byte LDS read.  dS goes to LDS row-major (one row
// per query) after an exchange between lanes that gives every lane 8 consecutive keys of one
// query, so the A operand of dQ = dS K is a 16-byte read as well.  LDS measurements on gfx950
// put 16-byte accesses at ~121 B/clk per CU and every 8-byte access (transposing reads
// included) at ~40 B/clk.
// ------------------------------------------------------------------------------------------
template <int DQK, int DV, int TM_>
struct MainTile {
  static constexpr int TM = TM_;       // query rows per block (32 or 64)
  static constexpr int MT = TM / 32;   // 32-row MFMA tiles per block
  static constexpr int TN = 128;       // keys per tile
  static constexpr int QS = DQK + 8;   // row-major strides in elements (16-byte pad)
  static constexpr int OS = DV + 8;
  static constexpr int KS = DQK + 8;
  static constexpr int SR = TN + 8;    // dS rows (one per query)
  static constexpr int TS = TM + 8;    // transposed copies: one row per head-dim column
  // staging blocks of RB query rows x 8 columns, one per thread and step; 8-row blocks give
  // 16-byte transposed writes and are used whenever the Q blocks fill whole waves
  static constexpr int RB = ((TM / 8) * (DQK / 8)) % 64 == 0 ? 8 : 4;
  static constexpr int QBLK = (TM / RB) * (DQK / 8);  // staging blocks of Q
  static constexpr int OBLK = (TM / RB) * (DV / 8);   // ... of dO (ids after Q's)
  static constexpr int NV = (QBLK + OBLK + 255) / 256;  // blocks per thread
  static constexpr int NT = MT * (DQK / 32);            // 32x32 tiles of a dQ block
  static constexpr int NTW = (NT + 3) / 4;              // dQ tiles per wave
  // every dQ tile of a wave (tiles wave + 4*tt) uses the same 32 head-dim columns when the
  // DQK/32 column tiles divide 4: their K operand is kept in registers for the whole work item
  static constexpr bool KT_REGS = 4 % (DQK / 32) == 0 || NT <= 4;
  // a wave's staging blocks are all Q or all dO, so the choice of buffer is wave-uniform
  static_assert(QBLK % 64 == 0, "staging blocks of Q must fill whole waves");
};

// Position of query q (0 <= q < TM) inside a transposed row: bits 2 and 3 of q swapped, so
// that slots 0..7 of lane half h in reduction step ks are the 8 consecutive positions
// 16ks + 8h .. 16ks + 8h + 7.
__device__ __forceinline__ int tpos(int q) {
  return (q & ~12) | ((q & 4) << 1) | ((q & 8) >> 1);
}

// LDS row swizzles.  Row-major Q/dO copies keep row r at qrow(r) = r ^ ((r >> 4) & 3): the 8
// lanes of a staging write then hit 8 different 16-byte bank groups (plain rows 16 apart share
// one), and reads of 8 consecutive rows still do.  The dS tile keeps query row r at
// dsrow(r) = r ^ ((r & 8) >> 1), which does the same for the rows the dS exchange writes
// together (r, r+2, r+8, r+10) and for the dQ operand reads.  Both permute rows inside each
// aligned group of 16.
__device__ __forceinline__ int qrow(int r) { return r ^ ((r >> 4) & 3); }
__device__ __forceinline__ int dsrow(int r) { return r ^ ((r & 8) >> 1); }

// dS of one 32-query tile to LDS, one row per query.  On entry d[4c + e] is dS(query
// 8c + 4*hi + e of the tile, this lane's key).  Three exchanges move key bits into registers
// and query bits into lanes: lane bit 4 <-> e bit 0 (permlane16 swap, on fp32 values), then
// on bf16 pairs lane bit 0 <-> e bit 1 and lane bit 1 <-> c bit 0 (DPP).  Afterwards the lane
// holds, for c bit 1 = u, 8 consecutive keys 8*(lane bits 2,3) + 0..7 of query
// 16u + 8*(lane bit 1) + 4*hi + 2*(lane bit 0) + (lane bit 4), as one 16-byte row segment.
template <int SR>
__device__ __forceinline__ void write_ds_tile(uint16_t* ds_lds, const float (&d)[16], int row0,
                                              int col0, int lane) {
  unsigned w[4][2];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int e1 = 0; e1 < 2; ++e1) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(d[4 * c + 2 * e1]),
                                                      __float_as_uint(d[4 * c + 2 * e1 + 1]),
                                                      false, false);
      w[c][e1] = pack_bf16(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
  }
  const bool x0 = (lane & 1) != 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const unsigned t0 = xor1(w[c][0]);
    const unsigned t1 = xor1(w[c][1]);
    const unsigned n0 = x0 ? t1 : w[c][0];
    const unsigned n1 = x0 ? w[c][1] : t0;
    w[c][0] = n0;
    w[c][1] = n1;
  }
  const bool x1 = (lane & 2) != 0;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const unsigned a = w[2 * u][s];
      const unsigned b = w[2 * u + 1][s];
      const unsigned ta = xor2(a);
      const unsigned tb = xor2(b);
      w[2 * u][s] = x1 ? tb : a;
      w[2 * u + 1][s] = x1 ? b : ta;
    }
  }
  const int row = row0 + 8 * ((lane >> 1) & 1) + 4 * (lane >> 5) + 2 * (lane & 1) + ((lane >> 4) & 1);
  const int col = col0 + 8 * ((lane >> 2) & 3);
#pragma unroll
  for (int u = 0; u < 2; ++u)
    *(u32x4*)&ds_lds[dsrow(row + 16 * u) * SR + col] = u32x4{w[2 * u][0], w[2 * u][1], w[2 * u + 1][0], w[2 * u + 1][1]};
}

// Query row of register u of a staging block whose first row is r0.  8-row blocks hold rows
// r0 + {0..3, 8..11} (r0 = 16a + 4b), which are 8 consecutive transposed positions.
template <int RB>
__device__ __forceinline__ int block_row(int r0, int u) {
  return RB == 8 ? r0 + (u & 3) + 8 * (u >> 2) : r0 + u;
}

// Write one staging block (RB rows of x, column chunk c8) into a row-major tile and into the
// transposed copy, where its rows occupy positions pos0 .. pos0 + RB - 1.
template <int RB, int TSS>
__device__ __forceinline__ void stage_block(uint16_t* rm, uint16_t* tr, int RS,
                                            const u32x4 (&x)[RB], int r0, int pos0, int c8) {
#pragma unroll
  for (int u = 0; u < RB; ++u) *(u32x4*)&rm[qrow(block_row<RB>(r0, u)) * RS + c8 * 8] = x[u];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // columns 2k (low halves) and 2k+1 (high halves), rows in position order
    unsigned lo[RB / 2], hi[RB / 2];
#pragma unroll
    for (int t = 0; t < RB / 2; ++t) {
      lo[t] = __builtin_amdgcn_perm(x[2 * t + 1][k], x[2 * t][k], 0x05040100u);
      hi[t] = __builtin_amdgcn_perm(x[2 * t + 1][k], x[2 * t][k], 0x07060302u);
    }
    if constexpr (RB == 8) {
      *(u32x4*)&tr[(c8 * 8 + 2 * k) * TSS + pos0] = u32x4{lo[0], lo[1], lo[2], lo[3]};
      *(u32x4*)&tr[(c8 * 8 + 2 * k + 1) * TSS + pos0] = u32x4{hi[0], hi[1], hi[2], hi[3]};
    } else {
      *(u32x2*)&tr[(c8 * 8 + 2 * k) * TSS + pos0] = u32x2{lo[0], lo[1]};
      *(u32x2*)&tr[(c8 * 8 + 2 * k + 1) * TSS + pos0] = u32x2{hi[0], hi[1]};
    }
  }
}

// DQM: 0 = fp32 atomic adds, 1 = deterministic fp32 splits, 2 = packed bf16 atomic adds.
// X: bit 0 = an additive bias, bit 1 = dropout.  The bias joins the logits (an absent bias
// reads zeros from an empty resource) and dS goes to dbias or its full-shape scratch when
// that is requested; dropout's keep mask comes from Philox behind one uniform branch (so the
// bias instance serves bias with or without dropout).
template <int DQK, int DV, int TM_, int DQM, int X>
__global__ __launch_bounds__(256, 1) void k_bwd_main(const KParams p) {
  constexpr bool XB = (X & 1) != 0;
  constexpr bool XD = (X & 2) != 0;
  constexpr bool DET = DQM == 1;
  using T = MainTile<DQK, DV, TM_>;
  constexpr int TM = T::TM, MT = T::MT, TN = T::TN, QS = T::QS, OS = T::OS, KS = T::KS,
                SR = T::SR, TS = T::TS, NT = T::NT, RB = T::RB;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[TN * KS];    // K_j, row-major
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[TM * QS];    // Q_i, row-major
  __shared__ __attribute__((aligned(16))) uint16_t o_lds[TM * OS];    // dO_i, row-major
  __shared__ __attribute__((aligned(16))) uint16_t qt_lds[DQK * TS];  // Q_i transposed
  __shared__ __attribute__((aligned(16))) uint16_t ot_lds[DV * TS];   // dO_i transposed
  __shared__ __attribute__((aligned(16))) uint16_t ds_lds[TM * SR];   // dS (query-major)
  __shared__ __attribute__((aligned(16))) float lse_lds[256];        // LSE_i * log2(e)
  __shared__ __attribute__((aligned(16))) float dd_lds[256];         // D_i
  // bias instances: each wave's 32 keys of the step's bias rows, keys in lane order
  __shared__ __attribute__((aligned(16))) uint16_t bias_lds[XB && DQK <= 128 ? 4 * TM * 32 : 8];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int g16 = lane >> 4;
  const int i16 = lane & 15;

  const int nbh = p.Hkv * p.B;
  // work group -> (item, part, head): item-major, so causal items with the most work start
  // first; part `part` of kv_parts takes its share of the item's steps
  const int ip = blockIdx.x / nbh;
  const int item = ip / p.kv_parts;  // key tiles item*T .. item*T + T - 1; split `item`
  const int part = ip - item * p.kv_parts;
  const int rem = blockIdx.x - ip * nbh;
  const int g = rem % p.Hkv;
  const int b = rem / p.Hkv;
  const bool group = p.seqstart_q != nullptr;
  const Seg sg = seg_of(p, b);
  const MaskGeom mg = mask_geom(p.mask_type, p.window_left, p.window_right, sg.lq, sg.lk);
  // query blocks whose partial this item has already written into its split (a contiguous
  // range: consecutive tiles touch overlapping or adjacent ranges)
  int64_t w_lo = 1, w_hi = 0;
  // Parts own steps (query head h, query block qb) of the union of the item's tiles' query
  // block ranges [u_lo, u_hi], numbered h-major: union step u = (h - g*group_size) * nbu +
  // qb - u_lo, part `part` owning u in [nu*part/kv_parts, nu*(part+1)/kv_parts).  Ownership
  // does not depend on the tile, so the split blocks a part reads back on a later tile are
  // exactly the ones it wrote itself.
  int64_t u_lo = 1, u_hi = 0;
  for (int tsub = 0; tsub < p.tiles_per_item; ++tsub) {
    const int j = item * p.tiles_per_item + tsub;
    if ((int64_t)j * TN >= sg.lk) break;
    int64_t lo, hi;
    qblocks_for_tile(mg, sg.lq, sg.lk, j, TM, TN, &lo, &hi);
    if (hi >= lo) {
      const bool had = u_hi >= u_lo;
      u_lo = had ? min(u_lo, lo) : lo;
      u_hi = had ? max(u_hi, hi) : hi;
    }
  }
  const int64_t nbu = u_hi >= u_lo ? u_hi - u_lo + 1 : 0;
  const int64_t nu = nbu * p.group_size;
  const int64_t u_a = nu * part / p.kv_parts;
  const int64_t u_e = nu * (part + 1) / p.kv_parts;
  for (int tsub = 0; tsub < p.tiles_per_item; ++tsub) {
  const int j = item * p.tiles_per_item + tsub;
  const int64_t key0 = (int64_t)j * TN;
  if (key0 >= sg.lk) break;  // the rest of the item is beyond this segment (uniform)
  if (tsub > 0) {
    __builtin_amdgcn_s_waitcnt(0);  // the previous tile's partial stores have completed
    __syncthreads();                // every wave is done with the previous tile's LDS
  }
  const int nk = (int)min((int64_t)TN, sg.lk - key0);
  int64_t qb_lo, qb_hi;
  qblocks_for_tile(mg, sg.lq, sg.lk, j, TM, TN, &qb_lo, &qb_hi);
  const int nblk = qb_hi >= qb_lo ? (int)(qb_hi - qb_lo + 1) : 0;
  const int nsteps = nblk * p.group_size;
  // allowed  <=>  lo_d <= key - row <= hi_d (and both inside the segment).  key - row always
  // lies in [-lq, lk], so the bounds are clamped to that range and the test becomes one
  // unsigned compare: (unsigned)(key - row - lo_d) <= span.
  const int64_t lo64 = mg.left >= 0 ? mg.delta - mg.left : -sg.lq;
  const int64_t hi64 = mg.right >= 0 ? mg.delta + mg.right : sg.lk;
  const int lo_d = (int)max(lo64, -sg.lq);
  const int hi_d = (int)min(hi64, sg.lk);
  const unsigned span = (unsigned)(hi_d - lo_d);  // only used when some pair is allowed

  const int tr_row = i16 >> 2;                        // row inside a 4-row transpose block
  const int tr_col = 16 * (g16 & 1) + 4 * (i16 & 3);  // column offset inside a 32-wide tile

  // K tile -> LDS (row-major); the wave's V rows -> registers (B operand of dP).
  const int key_l = wave * 32 + kmap(l32);
  const bool key_ok = key_l < nk;
  // bias rows start 16-byte aligned and no 8-key chunk straddles Sk (the bias staging below)
  const bool bias_rows16 = XB && ((uintptr_t)p.bias & 15u) == 0 &&
                           ((p.bias_s[0] | p.bias_s[1] | p.bias_s[2]) & 7) == 0 && (p.Sk & 7) == 0;
  bf16x8 vw[DV / 16];
  {
    const int64_t krow = sg.k_row0 + key0 + (key_ok ? key_l : 0);
    const uint16_t* kp = p.k + elem_off(p.k_s, group, b, krow, g);
    const uint16_t* vp = p.v + elem_off(p.v_s, group, b, krow, g);
#pragma unroll
    for (int kk = 0; kk < DQK / 16; ++kk) {
      const bf16x8 x = *(const bf16x8*)(kp + 16 * kk + 8 * hi);
      *(bf16x8*)&k_lds[key_l * KS + 16 * kk + 8 * hi] = key_ok ? x : bf16x8{};
    }
#pragma unroll
    for (int kk = 0; kk < DV / 16; ++kk) {
      const bf16x8 x = *(const bf16x8*)(vp + 16 * kk + 8 * hi);
      vw[kk] = key_ok ? x : bf16x8{};
    }
  }
  __syncthreads();

  // The wave's K rows as the B operand of S, kept in registers for the whole work item.
  bf16x8 kf[DQK / 16];
#pragma unroll
  for (int kk = 0; kk < DQK / 16; ++kk) kf[kk] = *(const bf16x8*)&k_lds[key_l * KS + 16 * kk + 8 * hi];

  // dQ work of this wave: tiles ti = wave + 4*tt (tt < NTW) of the MT x (DQK/32) grid.  With
  // KT_REGS the wave's K operand (its 32 head-dim columns over the tile's keys) is read once.
  bf16x8 kt[T::KT_REGS ? TN / 16 : 1];
  if (T::KT_REGS) {
    const int nd = wave % (DQK / 32);
#pragma unroll
    for (int kk = 0; kk < TN / 16; ++kk) {
      const int kb = 16 * kk + 8 * hi + tr_row;
      kt[kk] = tr_read(&k_lds[kb * KS + 32 * nd + tr_col], &k_lds[(kb + 4) * KS + 32 * nd + tr_col]);
    }
  }

  f32x16 dk_acc[DQK / 32];
  f32x16 dv_acc[DV / 32];
#pragma unroll
  for (int n = 0; n < DQK / 32; ++n) dk_acc[n] = f32x16{};
#pragma unroll
  for (int n = 0; n < DV / 32; ++n) dv_acc[n] = f32x16{};

  // ---- prefetch registers for one step: RB-row x 8-column blocks of Q and dO, LSE2, D ----
  // Block ids tid + 256v: ids below QBLK are Q blocks, the next OBLK are dO blocks; block id
  // covers row group id % (TM/RB) and column chunk id / (TM/RB).  Buffer loads over the
  // block's valid rows return zeros for rows past the segment end (and for everything when
  // the step does not exist, whose resources are empty).  The registers are not touched until
  // they are written to LDS, so nothing waits for the loads before then.  Offsets inside a
  // block are 32-bit (the plan bounds the sequence strides).
  u32x4 pre[T::NV][RB];
  // deterministic mode, later tiles of an item: the item's partial of the step's query block
  // (written by an earlier tile) is read back during the step and added before the store
  u32x4 prev[T::NTW][4];
  float lpre = 0.f, dpre = 0.f;
  const int qs1 = (int)p.q_s[1];
  const int os1 = (int)p.do_s[1];
  auto blk_geom = [&](int id, int& r0, int& pos0, int& c8) {
    const int rg = id % (TM / RB);
    c8 = id / (TM / RB);
    if (RB == 8) {
      r0 = 16 * (rg >> 1) + 4 * (rg & 1);
      pos0 = 8 * rg;
    } else {
      r0 = 4 * rg;
      pos0 = tpos(r0);
    }
  };
  int nq_pre = 0;  // valid rows of the prefetched step
  auto load_step = [&](bool valid, int h, int64_t q0) {
    const int nq = valid ? (int)min((int64_t)TM, sg.lq - q0) : 0;
    nq_pre = nq;
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(
        p.q + (valid ? elem_off(p.q_s, group, b, sg.q_row0 + q0, h) : 0),
        nq > 0 ? (uint32_t)((nq - 1) * qs1 + DQK) * 2u : 0u);
    const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(
        p.dout + (valid ? elem_off(p.do_s, group, b, sg.q_row0 + q0, h) : 0),
        nq > 0 ? (uint32_t)((nq - 1) * os1 + DV) * 2u : 0u);
#pragma unroll
    for (int v = 0; v < T::NV; ++v) {
      const int id0 = tid + 256 * v;
      if ((T::QBLK + T::OBLK) % 256 == 0 || id0 < T::QBLK + T::OBLK) {
        const bool isq = __builtin_amdgcn_readfirstlane(id0) < T::QBLK;  // wave-uniform
        const int id = isq ? id0 : id0 - T::QBLK;
        const __amdgpu_buffer_rsrc_t rs = isq ? rq : ro;
        const int st = isq ? qs1 : os1;
        int r0, pos0, c8;
        blk_geom(id, r0, pos0, c8);
#pragma unroll
        for (int u = 0; u < RB; ++u)
          pre[v][u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (block_row<RB>(r0, u) * st + c8 * 8) * 2, 0, 0);
      }
    }
    const int64_t row0 = valid ? (int64_t)h * p.rows_q + sg.ws_row0 + q0 : 0;
    lpre = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(p.lse2 + row0, (uint32_t)nq * 4u), tid * 4, 0, 0));
    dpre = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(p.dsum + row0, (uint32_t)nq * 4u), tid * 4, 0, 0));
  };
  auto store_step = [&]() {
#pragma unroll
    for (int v = 0; v < T::NV; ++v) {
      const int id0 = tid + 256 * v;
      if ((T::QBLK + T::OBLK) % 256 == 0 || id0 < T::QBLK + T::OBLK) {
        const bool isq = __builtin_amdgcn_readfirstlane(id0) < T::QBLK;  // wave-uniform
        const int id = isq ? id0 : id0 - T::QBLK;
        int r0, pos0, c8;
        blk_geom(id, r0, pos0, c8);
        stage_block<RB, TS>(isq ? q_lds : o_lds, isq ? qt_lds : ot_lds, isq ? QS : OS, pre[v], r0,
                            pos0, c8);
      }
    }
    // rows past the segment end get LSE = +inf, so their P is exactly 0
    lse_lds[tid] = tid < nq_pre ? lpre : __builtin_inff();
    dd_lds[tid] = dpre;
  };

  // The arithmetic of one step between its two barriers: S, dP, then per 32-query tile P, dS,
  // the dV/dK products and the dS tile to LDS (so the exponentials of one tile can overlap
  // the products of the other).
  auto compute_step = [&](int q0, int hq) {
    // bias of the lane's (query, key) pairs, issued before the products that hide its latency;
    // register 16m + r pairs with the S/dP result register r of row tile m.  Rows past the
    // plane are outside the resource (zeros); keys past the tile end are masked below.
    // With 16-byte aligned bias rows and Sk a multiple of 8 the wave loads its 32 keys of
    // the step's rows as 16-byte chunks (no chunk straddles Sk or the plane end), stages
    // them in its own LDS region with the keys in lane order, and reads them back with
    // transposing reads that give each lane its key for 4 rows at once; otherwise (and at
    // d_qk = 192, whose registers have no room for the chunks) one 2-byte load per value.
    constexpr bool kStage = XB && DQK <= 128;
    constexpr bool kVecOnly = XB && DQK == 128 && TM == 64;  // the plan takes it only when aligned
    float bv[XB && !kVecOnly ? MT * 16 : 1];
    u32x4 braw[kStage ? TM / 16 : 1];
    const bool bias_vec = kStage && (kVecOnly || bias_rows16);
    if constexpr (XB) {
      const __amdgpu_buffer_rsrc_t rb =
          buffer_rsrc(p.bias + (int64_t)b * p.bias_s[0] + (int64_t)hq * p.bias_s[1], p.bias_plane_bytes);
      const int bs2 = (int)p.bias_s[2];
      if (kStage && bias_vec) {
#pragma unroll
        for (int c = 0; c < TM / 16; ++c) {
          const int qc = lane + 64 * c;  // chunk qc: row qc / 4, keys 8 * (qc % 4) .. + 7
          braw[c] = __builtin_amdgcn_raw_buffer_load_b128(
              rb, ((q0 + (qc >> 2)) * bs2 + (int)key0 + 32 * wave + 8 * (qc & 3)) * 2, 0, 0);
        }
      } else if constexpr (!kVecOnly) {
        const int col = (int)key0 + key_l;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = q0 + 32 * m + 8 * (r >> 2) + 4 * hi + (r & 3);
            const unsigned short x = __builtin_amdgcn_raw_buffer_load_b16(rb, (row * bs2 + col) * 2, 0, 0);
            bv[16 * m + r] = __uint_as_float((unsigned)x << 16);
          }
      }
    }
    const __amdgpu_buffer_rsrc_t rdb = buffer_rsrc(
        XB && p.dbias_acc != nullptr ? p.dbias_acc + ((int64_t)b * p.Hq + hq) * p.Sq * p.Sk : nullptr,
        XB && p.dbias_acc != nullptr ? (uint32_t)p.Sq * (uint32_t)p.Sk * 4u : 0u);
    f32x16 s_acc[MT];
    f32x16 dp_acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      s_acc[m] = f32x16{};
      dp_acc[m] = f32x16{};
    }
    // ---- S = Q_i K_w^T and dP = dO_i V_w^T (MT row tiles of 32 queries) ----
    // all operands of a row tile are read before its products, so the reads overlap
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      bf16x8 qa[DQK / 16], oa[DV / 16];
#pragma unroll
      for (int kk = 0; kk < DQK / 16; ++kk)
        qa[kk] = *(const bf16x8*)&q_lds[qrow(32 * m + l32) * QS + 16 * kk + 8 * hi];
#pragma unroll
      for (int kk = 0; kk < DV / 16; ++kk)
        oa[kk] = *(const bf16x8*)&o_lds[qrow(32 * m + l32) * OS + 16 * kk + 8 * hi];
#pragma unroll
      for (int kk = 0; kk < DQK / 16; ++kk) s_acc[m] = mfma(qa[kk], kf[kk], s_acc[m]);
#pragma unroll
      for (int kk = 0; kk < DV / 16; ++kk) dp_acc[m] = mfma(oa[kk], vw[kk], dp_acc[m]);
    }
    if constexpr (kStage) {
      if (bias_vec) {
        // key k of the wave's 32 goes to position 16 * (k % 2) + k / 2 of its row, the inverse
        // of kmap, so lane l finds its key at position l % 32
        uint16_t* bw = &bias_lds[wave * TM * 32];
#pragma unroll
        for (int c = 0; c < TM / 16; ++c) {
          const int qc = lane + 64 * c, row = qc >> 2, j = qc & 3;
          const u32x4 x = braw[c];
          *(u32x2*)&bw[row * 32 + 4 * j] =
              u32x2{(x[0] & 0xFFFFu) | (x[1] << 16), (x[2] & 0xFFFFu) | (x[3] << 16)};
          *(u32x2*)&bw[row * 32 + 16 + 4 * j] =
              u32x2{(x[0] >> 16) | (x[1] & 0xFFFF0000u), (x[2] >> 16) | (x[3] & 0xFFFF0000u)};
        }
      }
    }
    // mask: pair (row, key) allowed iff (unsigned)(key - row - lo_d) <= span; keys past the
    // tile end get an offset that fails for every row of the block
    const int t0 = key_ok ? (int)(key0 - q0) + key_l - lo_d - 4 * hi : (int)span + TM + 1;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      // ---- P, dS of tile m: register r holds query 32m + 8(r/4) + 4*hi + r%4 ----
      bf16x8 pa[2], sa[2];
      float ds32[16];
      // the bias of tile m: rows 32m + 8u + 4hi + e of the lane's key (staged: lane s of a
      // 16-lane group points at row s / 4 of the 4-row block and its positions 4 (s % 4) .. + 3
      // of the group's 16)
      float bm[XB ? 16 : 1];
      if constexpr (XB) {
        if (kStage && bias_vec) {
          const uint16_t* bw = &bias_lds[wave * TM * 32];
          const int i16 = lane & 15;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)&bw[
                (32 * m + 8 * u + 4 * hi + (i16 >> 2)) * 32 + 16 * (g16 & 1) + 4 * (i16 & 3)]);
#pragma unroll
            for (int e = 0; e < 4; ++e) bm[4 * u + e] = __uint_as_float((unsigned)(unsigned short)t[e] << 16);
          }
        } else if constexpr (!kVecOnly) {
#pragma unroll
          for (int r = 0; r < 16; ++r) bm[r] = bv[16 * m + r];
        }
      }
      // dropout: the tile's rows 32m + 8c + 4hi + (0..3) of this lane's key take bytes
      // (key % 4) of the Philox output for (key / 4, row / 4).  The four lanes of one key
      // quad (l, l^1, l^16, l^17: key bits 0-1 are lane bits 4 and 0) need the same four
      // outputs (c = 0..3); each computes one (c = its position t in the group), transposes
      // it to four per-key words of 4 row bytes, and the group trades them.
      unsigned zw[4] = {~0u, ~0u, ~0u, ~0u};  // per c: keep bytes of rows e = 0..3
      if constexpr (XD) {
        if (p.drop_k < 256) {
          const unsigned kpos = (unsigned)(key0 + key_l);
          const unsigned t = (unsigned)(lane & 1) | ((unsigned)(lane >> 4) & 1u) << 1;
          unsigned w[4] = {kpos >> 2, (unsigned)(q0 + 32 * m + 8 * (int)t + 4 * hi) >> 2,
                           (unsigned)(b * p.Hq + hq), p.offset_lo};
          philox4x32_10(w, p.seed_lo, p.seed_hi);
          unsigned tw[4];
          byte_transpose4(w, tw);  // tw[k]: the 4 row bytes of key k % 4
          // round u: the lane at group position t ^ u sends what this lane needs
          const unsigned kswap0 = ((t >> 1) & 1u) | ((t & 1u) << 1);  // key byte of position t
          unsigned r[4];
          r[0] = sel4(tw, kswap0);
          {
            const unsigned pu = t ^ 1u, ku = ((pu >> 1) & 1u) | ((pu & 1u) << 1);
            r[1] = xor1(sel4(tw, ku));
          }
          {
            const unsigned pu = t ^ 2u, ku = ((pu >> 1) & 1u) | ((pu & 1u) << 1);
            r[2] = xor16(sel4(tw, ku), lane);
          }
          {
            const unsigned pu = t ^ 3u, ku = ((pu >> 1) & 1u) | ((pu & 1u) << 1);
            r[3] = xor16(xor1(sel4(tw, ku)), lane);
          }
#pragma unroll
          for (int c = 0; c < 4; ++c) zw[c] = sel4(r, t ^ (unsigned)c);
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int qr = 32 * m + 8 * c + 4 * hi;
        const f32x4 l4 = *(const f32x4*)&lse_lds[qr];
        const f32x4 d4 = *(const f32x4*)&dd_lds[qr];
        float zf[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (XD) {
          if (p.drop_k < 256) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              zf[e] = ((zw[c] >> (8 * e)) & 0xFFu) < (unsigned)p.drop_k ? p.drop_scale : 0.f;
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * c + e;
          float xl = s_acc[m][r] * p.scale_log2 - l4[e];
          if constexpr (XB) xl = __builtin_fmaf(bm[r], kLog2e, xl);
          float pv = __builtin_amdgcn_exp2f(xl);
          pv = (unsigned)(t0 - (32 * m + 8 * c + e)) <= span ? pv : 0.f;
          const float dsv = pv * (dp_acc[m][r] * zf[e] - d4[e]);
          pa[c >> 1][(c & 1) * 4 + e] = (__bf16)(pv * zf[e]);
          sa[c >> 1][(c & 1) * 4 + e] = (__bf16)dsv;
          ds32[r] = dsv;
          if constexpr (XB) {
            // broadcast dbias: the full-shape fp32 dS, every (row, key) of the block, masked
            // pairs as 0; rows past the plane are dropped by the range check, keys past the
            // tile end skipped (a full-shape dbias is copied from the dS tile below)
            const unsigned drow = (unsigned)(q0 + 32 * m + 8 * c + 4 * hi + e);
            if (p.dbias_acc != nullptr && key_ok)
              __builtin_amdgcn_raw_buffer_store_b32(
                  __float_as_uint(dsv), rdb, (drow * (unsigned)p.Sk + (unsigned)(key0 + key_l)) * 4u, 0, 0);
          }
        }
      }
      // ---- dV += P^T dO_i ; dK += dS^T Q_i over this tile's queries ----
      // reduction step ks = 2m + t covers transposed positions 16ks .. 16ks + 15
      bf16x8 bo[2][DV / 32], bq[2][DQK / 32];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int n2 = 0; n2 < DV / 32; ++n2)
          bo[t][n2] = *(const bf16x8*)&ot_lds[(32 * n2 + l32) * TS + 16 * (2 * m + t) + 8 * hi];
#pragma unroll
        for (int n2 = 0; n2 < DQK / 32; ++n2)
          bq[t][n2] = *(const bf16x8*)&qt_lds[(32 * n2 + l32) * TS + 16 * (2 * m + t) + 8 * hi];
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int n2 = 0; n2 < DV / 32; ++n2) dv_acc[n2] = mfma(pa[t], bo[t][n2], dv_acc[n2]);
#pragma unroll
        for (int n2 = 0; n2 < DQK / 32; ++n2) dk_acc[n2] = mfma(sa[t], bq[t][n2], dk_acc[n2]);
      }
      write_ds_tile<SR>(ds_lds, ds32, 32 * m, 32 * wave, lane);
    }
  };

  // step n covers query head h = g*group_size + n / nblk and query block qb_lo + n % nblk;
  // this work group's part takes steps n0 .. n1 - 1: the tile's steps that come before union
  // step u number (u / nbu) * nblk + clamp(u_lo + u % nbu - qb_lo, 0, nblk)
  const auto steps_before = [&](int64_t u) -> int {
    if (nbu == 0) return 0;
    const int64_t c = min(max(u_lo + u % nbu - qb_lo, (int64_t)0), (int64_t)nblk);
    return (int)((u / nbu) * nblk + c);
  };
  const int n0 = steps_before(u_a);
  const int n1 = steps_before(u_e);
  int h = g * p.group_size + (nblk > 0 ? n0 / nblk : 0);
  int64_t q0 = (qb_lo + (nblk > 0 ? n0 % nblk : 0)) * TM;
  if (n1 > n0) {
    load_step(true, h, q0);
    store_step();
  }

  for (int n = n0; n < n1; ++n) {
    const int nq = (int)min((int64_t)TM, sg.lq - q0);
    int h_next = h;
    int64_t q0_next = q0 + TM;
    if (q0_next > qb_hi * TM) {
      q0_next = qb_lo * TM;
      ++h_next;
    }
    __syncthreads();  // LDS holds step n; every wave is done with step n-1's dS
    load_step(n + 1 < n1, h_next, q0_next);
    const __amdgpu_buffer_rsrc_t rdq = DET
        ? buffer_rsrc(p.dq_acc + (int64_t)item * p.split_stride + (int64_t)h * p.head_stride +
                          (sg.acc_row0 + q0) * DQK, (uint32_t)TM * DQK * 4u)
        : buffer_rsrc(p.dq_acc + (int64_t)h * p.head_stride + (sg.acc_row0 + q0) * DQK,
                      (uint32_t)nq * DQK * 4u);
    // bf16 mode: the step's block of slot (b, h) of the bf16 accumulator (rows = logical query
    // positions; the slot is padded to whole blocks, so the block is inside it)
    const __amdgpu_buffer_rsrc_t r16 =
        buffer_rsrc((const uint16_t*)p.dq_acc + (int64_t)b * p.split_stride + (int64_t)h * p.head_stride +
                        q0 * DQK, (uint32_t)TM * DQK * 2u);
    compute_step((int)q0, h);
    if (DET) {  // issued late: the S/dP accumulators are dead by now
      const int64_t qbn = q0 / TM;
      const __amdgpu_buffer_rsrc_t rprev =
          qbn >= w_lo && qbn <= w_hi ? rdq : buffer_rsrc(p.dq_acc, 0u);  // empty: reads 0
#pragma unroll
      for (int tt = 0; tt < T::NTW; ++tt) {
        const int ti = wave + 4 * tt;
        if (NT % 4 == 0 || ti < NT) {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            prev[tt][u] = __builtin_amdgcn_raw_buffer_load_b128(rprev, (ti * 1024 + u * 256 + lane * 4) * 4, 0, kPartialPolicy);
        }
      }
    }

    __syncthreads();  // dS complete; every wave is done reading this step's Q, dO tiles

    // full-shape dbias: the step's dS tile in LDS (bf16, masked pairs 0) is dbias for its
    // (row, key) pairs; 16-byte copies of 8 keys where dbias is aligned for them
    if constexpr (XB) {
      if (p.dbias_direct) {
        uint16_t* dplane = p.dbias + (int64_t)b * p.dbias_s[0] + (int64_t)h * p.dbias_s[1];
        const int64_t ds2 = p.dbias_s[2];
        const bool vec = (((uintptr_t)dplane | (uintptr_t)(ds2 * 2)) & 15u) == 0;
#pragma unroll
        for (int c = tid; c < TM * (TN / 8); c += 256) {
          const int row = c / (TN / 8), j = (int)key0 + 8 * (c % (TN / 8));
          const int64_t i = q0 + row;
          if (i < p.Sq && j < p.Sk) {
            const uint16_t* src = &ds_lds[dsrow(row) * SR + (j - (int)key0)];
            uint16_t* dst = dplane + i * ds2 + j;
            if (vec && j + 8 <= p.Sk) {
              *(u32x4*)dst = *(const u32x4*)src;
            } else {
              for (int e = 0; e < 8 && j + e < p.Sk; ++e) dst[e] = src[e];
            }
          }
        }
      }
    }

    // ---- dQ_i partial = dS K_j  (reduction over the tile's 128 keys) ----
    // Deterministic: the item's split block of this step (its own rows, padding included),
    // the earlier tiles' sum plus this tile's, per 32x32 tile as four 1 KB chunks (chunk u =
    // result registers 4u .. 4u+3 of every lane, lane order), so each 16-byte-per-lane store
    // or read-back covers one contiguous kilobyte.  Atomic:
    // fp32 adds into the row-major accumulator; the resource covers the block's valid rows,
    // so rows past the segment end are dropped (offsets go entirely in the per-lane operand:
    // the scalar offset is outside the range check).
#pragma unroll
    for (int tt = 0; tt < T::NTW; ++tt) {
      const int ti = wave + 4 * tt;
      if (NT % 4 == 0 || ti < NT) {
        const int mq = ti / (DQK / 32);
        const int nd = ti - mq * (DQK / 32);
        bf16x8 da[TN / 16];
#pragma unroll
        for (int kk = 0; kk < TN / 16; ++kk)
          da[kk] = *(const bf16x8*)&ds_lds[dsrow(32 * mq + l32) * SR + 16 * kk + 8 * hi];
        f32x16 acc = f32x16{};
#pragma unroll
        for (int kk = 0; kk < TN / 16; ++kk) {
          bf16x8 bk;
          if (T::KT_REGS) {
            bk = kt[kk];
          } else {
            const int kb = 16 * kk + 8 * hi + tr_row;
            bk = tr_read(&k_lds[kb * KS + 32 * nd + tr_col], &k_lds[(kb + 4) * KS + 32 * nd + tr_col]);
          }
          acc = mfma(da[kk], bk, acc);
        }
        if (DET) {
          const int voff = (ti * 1024 + lane * 4) * 4;
#pragma unroll
          for (int u = 0; u < 4; ++u)
            __builtin_amdgcn_raw_buffer_store_b128(
                u32x4{__float_as_uint(__uint_as_float(prev[tt][u][0]) + acc[4 * u]),
                      __float_as_uint(__uint_as_float(prev[tt][u][1]) + acc[4 * u + 1]),
                      __float_as_uint(__uint_as_float(prev[tt][u][2]) + acc[4 * u + 2]),
                      __float_as_uint(__uint_as_float(prev[tt][u][3]) + acc[4 * u + 3])},
                rdq, voff + 1024 * u, 0, kPartialPolicy);
        } else if (DQM == 2) {
          // packed bf16 adds.  Each lane packs rows (k, 8+k) of its column; lanes 2c and 2c+1
          // swap the packed words, and the even lane keeps row k of columns 2c, 2c+1, the odd
          // lane row 8+k.  The block is stored in this order: tile ti at 2048*ti bytes, the
          // words of register pair k2 at 256*k2, lane l's word at 4*l, so each atomic covers
          // 256 contiguous bytes.  Rows past the segment end add zeros (their P is 0) into the
          // slot's padding.  (No builtin exposes the buffer form of this atomic; it is written
          // out, without return value, so no wait depends on it.)
          const bool odd = (lane & 1) != 0;
          const unsigned sel = odd ? 0x03020706u : 0x05040100u;
#pragma unroll
          for (int k2 = 0; k2 < 8; ++k2) {
            const unsigned mine = pack_bf16(acc[k2], acc[8 + k2]);
            const unsigned other = xor1(mine);
            const unsigned v = __builtin_amdgcn_perm(other, mine, sel);
            const int voff = ti * 2048 + k2 * 256 + lane * 4;
            asm volatile("buffer_atomic_pk_add_bf16 %0, %1, %2, 0 offen" ::"v"(v), "v"(voff), "s"(r16));
          }
        } else {
          // register r holds query row 32mq + 8(r/4) + 4hi + r%4, column 32nd + l%32: each
          // atomic covers two 128-byte row segments
          const int voff = ((32 * mq + 4 * hi) * DQK + 32 * nd + l32) * 4;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
                acc[r], rdq, voff + (8 * (r >> 2) + (r & 3)) * DQK * 4, 0, 0);
        }
      }
    }
    store_step();  // this step's tiles are dead: stage step n+1 (zeros after the last step)
    h = h_next;
    q0 = q0_next;
  }

  // ---- epilogue: dK = scale * dK_acc, dV = dV_acc as bf16 (one part), or this part's fp32
  // partials (row kws_row0 + key of [part][g][rows_k][d_qk + d_v], unscaled).  Each lane holds
  // one column of 16 keys (result row i is the key 32*wave + kmap(i)), so the values go through
  // LDS: the wave writes a pass (one tensor in bf16, or half of its columns in fp32: at most
  // 2*d_qk bytes per key) into its 32 rows of the K tile and reads it back in 16-byte chunks,
  // which the buffer stores write as contiguous runs of each key's row; the stores' resources
  // span the tile's nk rows, so the range check drops keys past the tile end.  (2-byte stores
  // from the accumulator layout took about 35 cycles each.) ----
  __syncthreads();  // the last dQ products have read the K tile
  {
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int ln = lane_here();
    uint16_t* ep = &k_lds[32 * wave_s * KS];
    const auto pass = [&](const int which, const int half, const bool part_out) {
      const int nbt = which == 0 ? DQK / 32 : DV / 32;  // 32-column blocks of the tensor
      const int ncol = part_out ? nbt / 2 : nbt;        // ... in this pass
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 8 * (r >> 2) + 4 * (ln >> 5) + (r & 3);
#pragma unroll
        for (int n2 = 0; n2 < ncol; ++n2) {
          const int n = half * ncol + n2;
          const float v = which == 0 ? dk_acc[n][r] : dv_acc[n][r];
          if (!part_out)
            ep[m * KS + 32 * n2 + (ln & 31)] = to_bf16_bits(which == 0 ? v * p.scale : v);
          else
            *(float*)&ep[m * KS + 2 * (32 * n2 + (ln & 31))] = v;
        }
      }
      __amdgpu_buffer_rsrc_t rs;
      int row_bytes, col_bytes;
      if (!part_out) {
        const int64_t* st = which == 0 ? p.dk_s : p.dv_s;
        uint16_t* base = (which == 0 ? p.dk : p.dv) + elem_off(st, group, b, sg.k_row0 + key0, g);
        row_bytes = (int)st[1] * 2;
        col_bytes = 0;
        rs = buffer_rsrc(base, (uint32_t)((nk - 1) * (int)st[1] + (which == 0 ? DQK : DV)) * 2u);
      } else {
        float* base = p.dkv_acc + (((int64_t)part * p.Hkv + g) * p.rows_k + sg.kws_row0 + key0) * (DQK + DV);
        row_bytes = (DQK + DV) * 4;
        col_bytes = ((which == 0 ? 0 : DQK) + half * ncol * 32) * 4;
        rs = buffer_rsrc(base, (uint32_t)nk * (uint32_t)row_bytes);
      }
      const int nch = part_out ? 8 * ncol : 4 * nbt;  // 16-byte chunks per row in this pass
#pragma unroll
      for (int i = 0; i < nch / 2; ++i) {  // 32 rows * nch chunks over 64 lanes
        const int id = ln + 64 * i;
        const int row = id / nch, c = id - row * nch;
        const u32x4 x = *(const u32x4*)&ep[row * KS + 8 * c];
        const int voff = (32 * wave_s + kmap(row)) * row_bytes + col_bytes + 16 * c;
        if (part_out)
          __builtin_amdgcn_raw_buffer_store_b128(x, rs, voff, 0, kPartialPolicy);
        else
          __builtin_amdgcn_raw_buffer_store_b128(x, rs, voff, 0, 0);
      }
    };
    if (p.kv_parts == 1) {
      pass(0, 0, false);
      pass(1, 0, false);
    } else {
      pass(0, 0, true);
      pass(0, 1, true);
      pass(1, 0, true);
      pass(1, 1, true);
    }
  }
  if (nblk > 0) {
    const bool had = w_hi >= w_lo;
    w_lo = had ? min(w_lo, qb_lo) : qb_lo;
    w_hi = had ? max(w_hi, qb_hi) : qb_hi;
  }
  }  // tiles of the item
}

// ------------------------------------------------------------------------------------------
// Stage 3: dQ = bf16(scale * sum of the partials), one block of TM rows per work group.
// Deterministic mode sums, in ascending split order, exactly the key tiles whose rows meet the
// block (qblocks_for_tile, as the main kernel) -- a contiguous range of tiles, since both ends
// of a tile's query range move monotonically with its keys; the next pair of splits is in
// flight while the current pair is added.
// ------------------------------------------------------------------------------------------
template <int DQK, int TM>
__device__ __forceinline__ void reduce_tiles(const KParams& p, const Seg& sg, bool group, int b,
                                             int h, int qb, int nq, int part) {
  const int TN = p.tile_n;
  constexpr int NT = (TM / 32) * (DQK / 32);   // 32x32 tiles per block
  constexpr int PPT = 1;                        // (tile, lane) pairs per thread
  const int tid = threadIdx.x + 256 * part;     // the block's pairs are split over work groups
  const MaskGeom mg = mask_geom(p.mask_type, p.window_left, p.window_right, sg.lq, sg.lk);
  const int ntiles = (int)((sg.lk + TN - 1) / TN);
  int jlo = 0, jhi = -1;
  for (int jt = 0; jt < ntiles; ++jt) {
    int64_t lo, hi;
    qblocks_for_tile(mg, sg.lq, sg.lk, jt, TM, TN, &lo, &hi);
    const bool in = qb >= lo && qb <= hi;
    if (in) {
      if (jhi < 0) jlo = jt;
      jhi = jt;
    } else if (jhi >= 0) {
      break;
    }
  }
  // split s holds key tiles s*T .. s*T + T - 1: the tile range maps to a split range
  const int T = p.tiles_per_item;
  if (jhi >= jlo) {
    jlo /= T;
    jhi /= T;
  }
  const float* base = p.dq_acc + (int64_t)h * p.head_stride + (sg.acc_row0 + (int64_t)qb * TM) * DQK;
  f32x4 acc[PPT][4];
#pragma unroll
  for (int pr = 0; pr < PPT; ++pr)
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[pr][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  // splits j, j+1 into x[0], x[1].  The loads are issued unconditionally, so the waits before
  // the adds count exactly the loads issued after them; a split past jhi has an empty
  // resource (loads return 0 and touch no memory) and is not added.
  auto load2 = [&](int j, f32x4 (&x)[2][PPT][4]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bool in = j + t <= jhi;
      const __amdgpu_buffer_rsrc_t r = buffer_rsrc(base + (in ? (int64_t)(j + t) * p.split_stride : 0),
                                                   in ? (uint32_t)(NT * 1024 * 4) : 0u);
#pragma unroll
      for (int pr = 0; pr < PPT; ++pr) {
        const int pair = tid + 256 * pr;
        if ((NT * 64) % 256 == 0 || pair < NT * 64) {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            x[t][pr][u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, ((pair >> 6) * 1024 + u * 256 + (pair & 63) * 4) * 4, 0, kPartialPolicy));
        }
      }
    }
  };
  auto add2 = [&](int j, const f32x4 (&x)[2][PPT][4]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (j + t > jhi) continue;
#pragma unroll
      for (int pr = 0; pr < PPT; ++pr)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[pr][u] += x[t][pr][u];
    }
  };
  // Two register buffers of two splits each take turns, so that the next pair of splits is
  // in flight while the current pair is added and no registers are copied between
  // iterations (a copy would make each iteration wait for the loads it has just issued).
  // The adds run in ascending split order.
  f32x4 xa[2][PPT][4], xb[2][PPT][4];
  if (jhi >= jlo) load2(jlo, xa);
  for (int jt = jlo; jt <= jhi; jt += 4) {
    load2(jt + 2, xb);
    add2(jt, xa);
    load2(jt + 4, xa);
    add2(jt + 2, xb);
  }
  // The work group's (up to) four 32x32 tiles go through LDS as bf16, so that each store
  // writes 16 bytes of a row and 16 consecutive threads cover 256 contiguous bytes of it.
  static_assert(PPT == 1, "one (tile, lane) pair per thread");
  __shared__ __attribute__((aligned(16))) uint16_t stage[4][32][40];  // [tile slot][row][col]
  const int64_t q0 = (int64_t)qb * TM;
  const int slot = threadIdx.x >> 6;
  if ((NT * 64) % 256 == 0 || tid < NT * 64) {
    const int ln = tid & 63;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        stage[slot][8 * u + 4 * (ln >> 5) + e][ln & 31] = to_bf16_bits(acc[0][u][e] * p.scale);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = threadIdx.x + 256 * k;  // 4 slots x 32 rows x 4 chunks of 8 columns
    const int row = c >> 4, sl = (c >> 2) & 3, ch = c & 3;
    const int ti = 4 * part + sl;
    if (ti < NT) {
      const int mq = ti / (DQK / 32), nd = ti % (DQK / 32);
      const int r = 32 * mq + row;
      if (r < nq)
        *(u32x4*)(p.dq + elem_off(p.dq_s, group, b, sg.q_row0 + q0 + r, h) + 32 * nd + 8 * ch) =
            *(const u32x4*)&stage[sl][row][8 * ch];
    }
  }
}

template <int DQK, int TM>
__device__ __forceinline__ void reduce_rows(const KParams& p, const Seg& sg, bool group, int b,
                                            int h, int qb, int nq) {
  constexpr int C4 = DQK / 4;                   // float4 chunks per row
  constexpr int PER = (TM * C4 + 255) / 256;    // chunks per thread
  const int tid = threadIdx.x;
  const int64_t q0 = (int64_t)qb * TM;
  const float* base = p.dq_acc + (int64_t)h * p.head_stride + (sg.acc_row0 + q0) * DQK;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int c = tid + 256 * u;
    const int r = c / C4;
    if (r < nq) {
      const f32x4 y = *(const f32x4*)(base + (int64_t)r * DQK + (c - r * C4) * 4) * p.scale;
      bf16x4 o;
      o[0] = (__bf16)y[0];
      o[1] = (__bf16)y[1];
      o[2] = (__bf16)y[2];
      o[3] = (__bf16)y[3];
      *(bf16x4*)(p.dq + elem_off(p.dq_s, group, b, sg.q_row0 + q0 + r, h) + (c - r * C4) * 4) = o;
    }
  }
}

// bf16 accumulator: slot (b, h), row = logical query position, each block of TM rows in the
// order the main kernel's packed atomics use: tile ti = (row/32)*(DQK/32) + col/32 at 1024*ti
// elements, and in it word w (elements 2w, 2w+1) = 64*k2 + l holds row 8*(r/4) + 4*(l/32) +
// r%4, r = k2 + 8*(l%2), of the tile, columns 2*((l%32)/2) and the next.  Read word by word
// (coalesced), written two dQ columns at a time.
template <int DQK, int TM>
__device__ __forceinline__ void convert_rows16(const KParams& p, const Seg& sg, bool group, int b,
                                               int h, int qb, int nq) {
  constexpr int WORDS = TM * DQK / 2;
  static_assert(WORDS % 256 == 0, "a block is a whole number of words per thread");
  constexpr int PER = WORDS / 256;
  const int tid = threadIdx.x;
  const int64_t q0 = (int64_t)qb * TM;
  const unsigned* base = (const unsigned*)((const uint16_t*)p.dq_acc + (int64_t)b * p.split_stride +
                                           (int64_t)h * p.head_stride + q0 * DQK);
  unsigned w[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) w[u] = base[tid + 256 * u];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int idx = tid + 256 * u;
    const int ti = idx >> 9, k2 = (idx >> 6) & 7, l = idx & 63;
    const int r = k2 + 8 * (l & 1);
    const int row = 32 * (ti / (DQK / 32)) + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
    const int col = 32 * (ti % (DQK / 32)) + 2 * ((l & 31) >> 1);
    if (row < nq) {
      const bf16x2 x = __builtin_bit_cast(bf16x2, w[u]);
      *(unsigned*)(p.dq + elem_off(p.dq_s, group, b, sg.q_row0 + q0 + row, h) + col) =
          pack_bf16((float)x[0] * p.scale, (float)x[1] * p.scale);
    }
  }
}

// Work groups per query block in deterministic mode: one per 256 (tile, lane) pairs.
template <int DQK, int TM>
constexpr int reduce_parts() { return ((TM / 32) * (DQK / 32) * 64 + 255) / 256; }

template <int DQK, int TM>
__global__ __launch_bounds__(256) void k_dq_reduce(const KParams p) {
  constexpr int PARTS = reduce_parts<DQK, TM>();
  const int part = p.deterministic ? (int)blockIdx.x % PARTS : 0;
  const int qb = p.deterministic ? (int)blockIdx.x / PARTS : (int)blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const bool group = p.seqstart_q != nullptr;
  const Seg sg = seg_of(p, b);
  const int64_t q0 = (int64_t)qb * TM;
  if (q0 >= sg.lq) return;
  const int nq = (int)min((int64_t)TM, sg.lq - q0);
  if (p.deterministic) {
    reduce_tiles<DQK, TM>(p, sg, group, b, h, qb, nq, part);
  } else if (p.dq_bf16) {
    convert_rows16<DQK, TM>(p, sg, group, b, h, qb, nq);
  } else {
    reduce_rows<DQK, TM>(p, sg, group, b, h, qb, nq);
  }
}

// ------------------------------------------------------------------------------------------
// dK = bf16(scale * sum of the parts' dK partials), dV = bf16(sum of the dV partials), in
// ascending part order.  One work group per (8 key rows, K/V head, segment), four values per
// thread and chunk; the loads of all parts of a chunk are issued before the sum.
// ------------------------------------------------------------------------------------------
constexpr int kDkvRows = 8;  // key rows per work group of k_dkv_reduce

template <int DQK, int DV>
__global__ __launch_bounds__(256) void k_dkv_reduce(const KParams p) {
  constexpr int W = DQK + DV;
  constexpr int C4 = W / 4;                              // float4 chunks per row
  constexpr int PER = (kDkvRows * C4 + 255) / 256;       // chunks per thread
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const bool group = p.seqstart_q != nullptr;
  const Seg sg = seg_of(p, b);
  const int64_t k0 = (int64_t)blockIdx.x * kDkvRows;
  if (k0 >= sg.lk) return;
  const int nk = (int)min((int64_t)kDkvRows, sg.lk - k0);
  const int64_t part_stride = (int64_t)p.Hkv * p.rows_k * W;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int c = threadIdx.x + 256 * u;
    const int r = c / C4;
    if (r < nk) {
      const int col = (c - r * C4) * 4;
      const int64_t krow = sg.k_row0 + k0 + r;
      const float* src = p.dkv_acc + ((int64_t)g * p.rows_k + sg.kws_row0 + k0 + r) * W + col;
      f32x4 part[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        part[q] = q < p.kv_parts ? __builtin_nontemporal_load((const f32x4*)(src + q * part_stride)) : f32x4{};
      f32x4 acc = part[0];
#pragma unroll
      for (int q = 1; q < 8; ++q)
        if (q < p.kv_parts) acc += part[q];
      bf16x4 o;
      if (col < DQK) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (__bf16)(acc[e] * p.scale);
        *(bf16x4*)(p.dk + elem_off(p.dk_s, group, b, krow, g) + col) = o;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (__bf16)acc[e];
        *(bf16x4*)(p.dv + elem_off(p.dv_s, group, b, krow, g) + (col - DQK)) = o;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// dbias = the full-shape dS summed over the bias's broadcast dimensions (ascending batch, then
// head, fp32), rounded to bf16.  One work group per (kDbiasRows query rows, output plane, 1024
// columns), four consecutive columns per thread (one 16-byte load per plane and row, one
// 8-byte store per row where dbias is aligned for it).  A (row, key) pair lies in a (query
// block, key tile) pair the main kernel skipped (no allowed pair there) exactly when
// qblocks_for_tile excludes the row's block; such entries were never written and count as 0,
// so the scratch needs no zeroing.
// ------------------------------------------------------------------------------------------
constexpr int kDbiasRows = 32;

__device__ __forceinline__ void store_bf16x4(uint16_t* dst, const float (&v)[4], int n, bool vec) {
  if (vec && n == 4) {
    *(u32x2*)dst = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u < n) dst[u] = to_bf16_bits(v[u]);
  }
}

__global__ __launch_bounds__(256) void k_dbias_reduce(const KParams p) {
  const int nchunk = (p.Sk + 1023) / 1024;
  const int i0 = ((int)blockIdx.x / nchunk) * kDbiasRows;  // first query row
  const int chunk = (int)blockIdx.x % nchunk;
  const int oh = blockIdx.y;                  // output head index (0 when broadcast)
  const int ob = blockIdx.z;                  // output batch index
  const int j0 = (chunk * 256 + (int)threadIdx.x) * 4;
  if (j0 >= p.Sk) return;
  const int n = min(4, p.Sk - j0);
  const int i1 = min(i0 + kDbiasRows, p.Sq);
  const MaskGeom mg = mask_geom(p.mask_type, p.window_left, p.window_right, p.Sq, p.Sk);
  int64_t lo, hi;
  qblocks_for_tile(mg, p.Sq, p.Sk, j0 / 128, p.tile_m, 128, &lo, &hi);  // j0..j0+3: one tile
  uint16_t* dst0 = p.dbias + (int64_t)ob * p.dbias_s[0] + (int64_t)oh * p.dbias_s[1] + j0;
  const int64_t ds2 = p.dbias_s[2];
  const bool vec = (((uintptr_t)dst0 | (uintptr_t)(ds2 * 2)) & 7u) == 0;
  const float zero[4] = {0.f, 0.f, 0.f, 0.f};
  if (p.dbias_direct) {  // written by the main kernel where seen; zeros elsewhere
    for (int i = i0; i < i1; ++i) {
      const int64_t qb = i / p.tile_m;
      if (qb < lo || qb > hi) store_bf16x4(dst0 + (int64_t)i * ds2, zero, n, vec);
    }
    return;
  }
  const int b0 = p.bias_b == 1 ? 0 : ob, b1 = p.bias_b == 1 ? p.B : ob + 1;
  const int h0 = p.bias_h == 1 ? 0 : oh, h1 = p.bias_h == 1 ? p.Hq : oh + 1;
  const int nh = h1 - h0, planes = (b1 - b0) * nh;
  const int64_t plane = (int64_t)p.Sq * p.Sk;
  const bool vload = (p.Sk & 3) == 0;  // rows of the fp32 scratch start 16-byte aligned
  for (int i = i0; i < i1; ++i) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const int64_t qb = i / p.tile_m;
    if (qb >= lo && qb <= hi) {
      const float* src0 = p.dbias_acc + (int64_t)i * p.Sk + j0;
      // the planes in ascending (batch, head) order; eight loads in flight
      for (int q = 0; q < planes; q += 8) {
        f32x4 x[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          x[t] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (q + t < planes) {
            const int bb = b0 + (q + t) / nh, hh = h0 + (q + t) % nh;
            const float* src = src0 + ((int64_t)bb * p.Hq + hh) * plane;
            if (vload && n == 4) {
              x[t] = *(const f32x4*)src;
            } else {
#pragma unroll
              for (int u = 0; u < 4; ++u)
                if (u < n) x[t][u] = src[u];
            }
          }
        }
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (q + t < planes)
#pragma unroll
            for (int u = 0; u < 4; ++u) acc[u] += x[t][u];
      }
    }
    store_bf16x4(dst0 + (int64_t)i * ds2, acc, n, vec);
  }
}

// ------------------------------------------------------------------------------------------
// Forward: O = softmax(scale * Q K^T + mask) V and LSE.  One work group per (block of 128
// queries, query head, segment); wave w owns queries 32w .. 32w+31 of the block.
//
// S^T = K Q^T puts one query per lane (lane l%32, in both lane halves) and, per 32-key block,
// 16 keys in the result registers, so the online softmax keeps its running max and sum per
// lane; the two lane halves hold different keys of the same query and agree on the max with
// one exchange.  P^T goes from the result registers straight into O^T += V^T P^T (V^T staged
// with keys in the order the registers feed the reduction slots, as the backward stages Q^T).
// Q stays in registers for the whole item; K (row-major) and V^T pass through LDS per 64-key
// tile, with the next tile's global loads in flight during the current one.
// ------------------------------------------------------------------------------------------
template <int DQK, int DV>
struct FwdTile {
  static constexpr int TQ = 128;                      // queries per block
  static constexpr int TK = 64;                       // keys per tile
  static constexpr int KS = DQK + 8;                  // K row-major stride (elements)
  static constexpr int VS = TK + 8;                   // V^T stride (one row per head-dim column)
  static constexpr int KBLK = (TK / 8) * (DQK / 8);   // 8x8 staging blocks of K
  static constexpr int VBLK = (TK / 8) * (DV / 8);    // ... of V (ids after K's)
  static constexpr int NV = (KBLK + VBLK + 255) / 256;
  static_assert(KBLK % 64 == 0, "staging blocks of K must fill whole waves");
};

template <int DQK, int DV, int X>
// X: bit 0 = bias, bit 1 = dropout (all four combinations are instances: the bias-and-dropout
// one does not fit two work groups per CU)
__global__ __launch_bounds__(256, DQK <= 128 && X != 3 ? 2 : 1) void k_fwd(const KParams p) {
  constexpr bool XB = (X & 1) != 0;
  constexpr bool XD = (X & 2) != 0;
  using T = FwdTile<DQK, DV>;
  constexpr int TQ = T::TQ, TK = T::TK, KS = T::KS, VS = T::VS;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[TK * KS];  // K tile, row-major
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[DV * VS];  // V tile, transposed

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int g = h / p.group_size;
  const bool group = p.seqstart_q != nullptr;
  const Seg sg = seg_of(p, b);
  // last query blocks first: under a causal mask they see the most keys
  const int64_t q0 = ((int64_t)gridDim.x - 1 - blockIdx.x) * TQ;
  if (q0 >= sg.lq) return;  // uniform
  const int nq = (int)min((int64_t)TQ, sg.lq - q0);
  const MaskGeom mg = mask_geom(p.mask_type, p.window_left, p.window_right, sg.lq, sg.lk);

  // keys any row of the block may see: [k_lo, k_hi]
  int64_t k_lo = 0, k_hi = sg.lk - 1;
  if (mg.left >= 0) k_lo = max(k_lo, q0 + mg.delta - mg.left);
  if (mg.right >= 0) k_hi = min(k_hi, q0 + nq - 1 + mg.delta + mg.right);
  const int t_lo = (int)(k_lo / TK);
  const int ntiles = k_hi >= k_lo ? (int)(k_hi / TK) - t_lo + 1 : 0;

  // this lane's query and its allowed key offsets: lo_l <= key - row <= hi_l
  const int row = (int)q0 + 32 * wave + l32;  // inside the segment; may be >= lq (not stored)
  int64_t lo_l = -(int64_t)row, hi_l = sg.lk - 1 - row;
  if (mg.left >= 0) lo_l = max(lo_l, mg.delta - mg.left);
  if (mg.right >= 0) hi_l = min(hi_l, mg.delta + mg.right);
  const bool lane_ok = hi_l >= lo_l && row < sg.lq;
  const unsigned span = lane_ok ? (unsigned)(hi_l - lo_l) : 0u;

  // Q rows of this wave as the B operand of S^T (rows past the segment end read as zeros)
  bf16x8 qf[DQK / 16];
  {
    const int qs1 = (int)p.q_s[1];
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(
        p.q + elem_off(p.q_s, group, b, sg.q_row0 + q0, h), (uint32_t)((nq - 1) * qs1 + DQK) * 2u);
#pragma unroll
    for (int kk = 0; kk < DQK / 16; ++kk)
      qf[kk] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                      rq, ((unsigned)(32 * wave + l32) * (unsigned)qs1 + 16u * kk + 8u * hi) * 2u, 0, 0));
  }

  // ---- staging: 8-row x 8-column blocks of K (row-major copy) and V (transposed copy) ----
  // K block id: column chunk fastest, so the 8 lanes of an LDS write group cover 8 chunks of
  // one row; V block id: row group fastest (8 consecutive transposed positions per lane group).
  u32x4 pre[T::NV][8];
  const int ks1 = (int)p.k_s[1];
  const int vs1 = (int)p.v_s[1];
  auto load_tile = [&](bool valid, int64_t kt0) {
    const int nk = valid ? (int)min((int64_t)TK, sg.lk - kt0) : 0;
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(
        p.k + (valid ? elem_off(p.k_s, group, b, sg.k_row0 + kt0, g) : 0),
        nk > 0 ? (uint32_t)((nk - 1) * ks1 + DQK) * 2u : 0u);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(
        p.v + (valid ? elem_off(p.v_s, group, b, sg.k_row0 + kt0, g) : 0),
        nk > 0 ? (uint32_t)((nk - 1) * vs1 + DV) * 2u : 0u);
#pragma unroll
    for (int v = 0; v < T::NV; ++v) {
      const int id0 = tid + 256 * v;
      if ((T::KBLK + T::VBLK) % 256 == 0 || id0 < T::KBLK + T::VBLK) {
        const bool isk = __builtin_amdgcn_readfirstlane(id0) < T::KBLK;  // wave-uniform
        if (isk) {
          const int c8 = id0 % (DQK / 8), r0 = 8 * (id0 / (DQK / 8));
#pragma unroll
          for (int u = 0; u < 8; ++u)
            pre[v][u] = __builtin_amdgcn_raw_buffer_load_b128(rk, ((r0 + u) * ks1 + c8 * 8) * 2, 0, 0);
        } else {
          const int id = id0 - T::KBLK;
          const int rg = id % (TK / 8), c8 = id / (TK / 8);
          const int r0 = 16 * (rg >> 1) + 4 * (rg & 1);
#pragma unroll
          for (int u = 0; u < 8; ++u)
            pre[v][u] = __builtin_amdgcn_raw_buffer_load_b128(
                rv, ((block_row<8>(r0, u)) * vs1 + c8 * 8) * 2, 0, 0);
        }
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int v = 0; v < T::NV; ++v) {
      const int id0 = tid + 256 * v;
      if ((T::KBLK + T::VBLK) % 256 == 0 || id0 < T::KBLK + T::VBLK) {
        const bool isk = __builtin_amdgcn_readfirstlane(id0) < T::KBLK;
        if (isk) {
          const int c8 = id0 % (DQK / 8), r0 = 8 * (id0 / (DQK / 8));
#pragma unroll
          for (int u = 0; u < 8; ++u) *(u32x4*)&k_lds[(r0 + u) * KS + c8 * 8] = pre[v][u];
        } else {
          const int id = id0 - T::KBLK;
          const int rg = id % (TK / 8), c8 = id / (TK / 8);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            unsigned lo[4], hi2[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              lo[t] = __builtin_amdgcn_perm(pre[v][2 * t + 1][k], pre[v][2 * t][k], 0x05040100u);
              hi2[t] = __builtin_amdgcn_perm(pre[v][2 * t + 1][k], pre[v][2 * t][k], 0x07060302u);
            }
            *(u32x4*)&vt_lds[(c8 * 8 + 2 * k) * VS + 8 * rg] = u32x4{lo[0], lo[1], lo[2], lo[3]};
            *(u32x4*)&vt_lds[(c8 * 8 + 2 * k + 1) * VS + 8 * rg] = u32x4{hi2[0], hi2[1], hi2[2], hi2[3]};
          }
        }
      }
    }
  };

  // ---- online softmax state (log2 units) and the O^T accumulator ----
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  f32x16 o_acc[DV / 32];
#pragma unroll
  for (int n = 0; n < DV / 32; ++n) o_acc[n] = f32x16{};

  if (ntiles > 0) {
    load_tile(true, (int64_t)t_lo * TK);
    store_tile();
  }
  // bias rows 8-byte aligned and Sk a multiple of 4 (the bias loads below)
  const bool bias_runs8 = XB && ((uintptr_t)p.bias & 7u) == 0 &&
                          ((p.bias_s[0] | p.bias_s[1] | p.bias_s[2]) & 3) == 0 && (p.Sk & 3) == 0;
  for (int it = 0; it < ntiles; ++it) {
    const int64_t kt0 = (int64_t)(t_lo + it) * TK;
    __syncthreads();  // LDS holds tile it
    load_tile(it + 1 < ntiles, kt0 + TK);

    // bias of this lane's query row for its keys of the tile, issued before the products;
    // rows past the plane read zeros, keys past the end are masked.  The lane's keys come in
    // runs of four consecutive ones (registers 4u .. 4u+3 of a block), one 8-byte load each
    // where the bias rows are 8-byte aligned and Sk is a multiple of 4 (no run straddles the
    // plane end); otherwise one 2-byte load per key.
    // bz[8kb + r/2] holds the bf16 bias of registers r (low half) and r+1 (high half), r even
    unsigned bz[XB ? 16 : 1];
    if constexpr (XB) {
      const __amdgpu_buffer_rsrc_t rb =
          buffer_rsrc(p.bias + (int64_t)b * p.bias_s[0] + (int64_t)h * p.bias_s[1], p.bias_plane_bytes);
      const int rowoff = row * (int)p.bias_s[2];
      if (bias_runs8) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const u32x2 w = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_raw_buffer_load_b64(rb, (rowoff + (int)kt0 + 32 * kb + 8 * u + 4 * hi) * 2, 0, 0));
            bz[8 * kb + 2 * u] = w[0];
            bz[8 * kb + 2 * u + 1] = w[1];
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const int k = rowoff + (int)kt0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
            const unsigned x0 = __builtin_amdgcn_raw_buffer_load_b16(rb, k * 2, 0, 0);
            const unsigned x1 = __builtin_amdgcn_raw_buffer_load_b16(rb, (k + 1) * 2, 0, 0);
            bz[8 * kb + r / 2] = x0 | (x1 << 16);
          }
      }
    }
    // S^T for the tile's two 32-key blocks: register r of block kb holds key
    // kt0 + 32kb + 8(r/4) + 4hi + r%4 of this lane's query
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x8 ka[DQK / 16];
#pragma unroll
      for (int kk = 0; kk < DQK / 16; ++kk)
        ka[kk] = *(const bf16x8*)&k_lds[(32 * kb + l32) * KS + 16 * kk + 8 * hi];
      s[kb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < DQK / 16; ++kk) s[kb] = mfma(ka[kk], qf[kk], s[kb]);
    }
    // mask and running max
    const int t0 = lane_ok ? (int)(kt0 - row - lo_l) + 4 * hi : (1 << 30);
    float mt = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ko = 32 * kb + 8 * (r >> 2) + (r & 3);
        float x = s[kb][r] * p.scale_log2;
        if constexpr (XB) {
          const unsigned w = bz[8 * kb + r / 2];
          x = __builtin_fmaf(__uint_as_float((r & 1) ? (w & 0xFFFF0000u) : (w << 16)), kLog2e, x);
        }
        s[kb][r] = (unsigned)(t0 + ko) <= span ? x : -__builtin_inff();
        mt = fmaxf(mt, s[kb][r]);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    // P (bf16, laid out as the B operand of O^T) and the running sum
    bf16x8 pb[2][2];
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // dropout (P in P V only; the running sum is of the full softmax): keys
      // kt0 + 32kb + 8c + 4hi .. +3 of this lane's row take word (row % 4) of the Philox
      // output for (key / 4, row / 4).  The four lanes of one row quad need the same four
      // outputs (c = 0..3): each computes one (c = row % 4) and the quad trades words.
      unsigned zw[4] = {~0u, ~0u, ~0u, ~0u};
      if constexpr (XD) {
        if (p.drop_k < 256) {
          const unsigned t = (unsigned)(lane & 3);  // == row % 4
          unsigned w[4] = {(unsigned)(kt0 + 32 * kb + 8 * (int)t + 4 * hi) >> 2, (unsigned)row >> 2,
                           (unsigned)(b * p.Hq + h), p.offset_lo};
          philox4x32_10(w, p.seed_lo, p.seed_hi);
          // round u: the lane at quad position t ^ u sends word t of its output
          const unsigned r[4] = {sel4(w, t), xor1(sel4(w, t ^ 1u)), xor2(sel4(w, t ^ 2u)),
                                 xor3(sel4(w, t ^ 3u))};
#pragma unroll
          for (int c = 0; c < 4; ++c) zw[c] = sel4(r, t ^ (unsigned)c);
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float zf[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (XD) {
          if (p.drop_k < 256) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              zf[e] = ((zw[c] >> (8 * e)) & 0xFFu) < (unsigned)p.drop_k ? p.drop_scale : 0.f;
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pv = __builtin_amdgcn_exp2f(s[kb][4 * c + e] - m_use);
          ls += pv;
          pb[kb][c >> 1][(c & 1) * 4 + e] = (__bf16)(pv * zf[e]);
        }
      }
    }
    l_run = l_run * alpha + ls;
    // O^T = alpha * O^T + V^T P^T (reduction step ks = 2kb + t covers transposed positions
    // 16ks .. 16ks + 15)
    bf16x8 va[4][DV / 32];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int n = 0; n < DV / 32; ++n)
        va[ks][n] = *(const bf16x8*)&vt_lds[(32 * n + l32) * VS + 16 * ks + 8 * hi];
#pragma unroll
    for (int n = 0; n < DV / 32; ++n) {
      o_acc[n] *= alpha;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) o_acc[n] = mfma(va[ks][n], pb[ks >> 1][ks & 1], o_acc[n]);
    }
    __syncthreads();  // every wave is done with tile it
    store_tile();     // tile it+1 (zeros after the last one)
  }

  // ---- finish: the lane halves' sums, O = O^T / l, LSE = (m + log2 l) * ln 2 ----
  const float l_all = l_run + __shfl_xor(l_run, 32);
  const float inv = l_all > 0.f ? 1.f / l_all : 0.f;
  if (row < sg.lq) {
    uint16_t* orow = p.o_out + elem_off(p.o_s, group, b, sg.q_row0 + row, h);
#pragma unroll
    for (int n = 0; n < DV / 32; ++n)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(o_acc[n][4 * c + e] * inv);
        *(bf16x4*)&orow[32 * n + 8 * c + 4 * hi] = v4;
      }
    if (hi == 0) {
      const float lse = l_all > 0.f ? (m_run + __builtin_log2f(l_all)) * 0.6931471805599453f
                                    : -__builtin_inff();
      p.lse_out[(group ? 0 : (int64_t)b * p.lse_s[0]) + (int64_t)h * p.lse_s[1] + sg.q_row0 + row] = lse;
    }
  }
}

__global__ __launch_bounds__(64) void k_header(uint64_t* ws, uint64_t magic, uint64_t fingerprint) {
  if (threadIdx.x == 0) {
    ws[0] = magic;
    ws[1] = fingerprint;
  }
}

// Zeroes n4 16-byte chunks (four per thread, each store instruction one contiguous 4 KiB run
// of the work group) and writes the workspace header from one lane, so the atomic modes'
// prepare step is a single launch.
__global__ __launch_bounds__(256) void k_zero(float* ptr, int64_t n4, uint64_t* ws, uint64_t magic,
                                              uint64_t fingerprint) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ws[0] = magic;
    ws[1] = fingerprint;
  }
  const int64_t stride = (int64_t)gridDim.x * 1024;
  for (int64_t i0 = (int64_t)blockIdx.x * 1024 + threadIdx.x; i0 < n4; i0 += stride) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (i0 + 256 * j < n4) ((f32x4*)ptr)[i0 + 256 * j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

}  // namespace

hipError_t launch_dot(const Plan& plan, const KParams& kp, hipStream_t stream) {
  // one more work group ranks the wide kernel's work groups when the plan orders them; it runs
  // even without query rows (keys only), since the main kernel still reads the list then
  if (plan.order_n > 2048 || (plan.order_n > 0 && kp.order == nullptr)) return hipErrorInvalidValue;
  const int64_t blocks = (plan.rows_q + kDotRows - 1) / kDotRows * plan.Hq + (plan.order_n > 0 ? 1 : 0);
  if (blocks == 0) return hipSuccess;
  if (plan.d_v == 64) {
    hipLaunchKernelGGL(k_dot<64>, dim3((unsigned)blocks), dim3(256), 0, stream, kp);
  } else {
    hipLaunchKernelGGL(k_dot<128>, dim3((unsigned)blocks), dim3(256), 0, stream, kp);
  }
  return hipGetLastError();
}

template <int DQK, int DV>
static void launch_fwd_t(const Plan& plan, const KParams& kp, dim3 grid, hipStream_t stream) {
  const int x = (plan.has_bias ? 1 : 0) | (plan.drop_k < 256 ? 2 : 0);
  if (x == 3) hipLaunchKernelGGL((k_fwd<DQK, DV, 3>), grid, dim3(256), 0, stream, kp);
  else if (x == 2) hipLaunchKernelGGL((k_fwd<DQK, DV, 2>), grid, dim3(256), 0, stream, kp);
  else if (x == 1) hipLaunchKernelGGL((k_fwd<DQK, DV, 1>), grid, dim3(256), 0, stream, kp);
  else hipLaunchKernelGGL((k_fwd<DQK, DV, 0>), grid, dim3(256), 0, stream, kp);
}

hipError_t launch_fwd(const Plan& plan, const KParams& kp, hipStream_t stream) {
  if (plan.B == 0 || plan.n_q_blocks == 0) return hipSuccess;
  const int64_t rows = (int64_t)plan.n_q_blocks * plan.tile_m;  // >= the longest segment
  const dim3 grid((unsigned)((rows + 127) / 128), (unsigned)plan.Hq, (unsigned)plan.B);
  if (plan.d_qk == 64) {
    launch_fwd_t<64, 64>(plan, kp, grid, stream);
  } else if (plan.d_qk == 128) {
    launch_fwd_t<128, 128>(plan, kp, grid, stream);
  } else {
    launch_fwd_t<192, 128>(plan, kp, grid, stream);
  }
  return hipGetLastError();
}

// WITH_BIAS = false for tile shapes the plan never uses with a bias (not compiled with one).
// Instances: X = 0 (plain), 2 (dropout), 3 (bias, with or without dropout).
template <int DQK, int DV, int TM, bool WITH_BIAS = true>
static void launch_main_t(const Plan& plan, const KParams& kp, dim3 grid, hipStream_t stream) {
  const int mode = plan.deterministic ? 1 : (plan.dq_bf16 ? 2 : 0);
  const bool drop = plan.drop_k < 256;
  if (WITH_BIAS && plan.has_bias) {
    if constexpr (WITH_BIAS) {
      if (mode == 1) hipLaunchKernelGGL((k_bwd_main<DQK, DV, TM, 1, 3>), grid, dim3(256), 0, stream, kp);
      else if (mode == 2) hipLaunchKernelGGL((k_bwd_main<DQK, DV, TM, 2, 3>), grid, dim3(256), 0, stream, kp);
      else hipLaunchKernelGGL((k_bwd_main<DQK, DV, TM, 0, 3>), grid, dim3(256), 0, stream, kp);
    }
  } else if (drop) {
    if (mode == 1) hipLaunchKernelGGL((k_bwd_main<DQK, DV, TM, 1, 2>), grid, dim3(256), 0, stream, kp);
    else if (mode == 2) hipLaunchKernelGGL((k_bwd_main<DQK, DV, TM, 2, 2>), grid, dim3(256), 0, stream, kp);
    else hipLaunchKernelGGL((k_bwd_main<DQK, DV, TM, 0, 2>), grid, dim3(256), 0, stream, kp);
  } else {
    if (mode == 1) hipLaunchKernelGGL((k_bwd_main<DQK, DV, TM, 1, 0>), grid, dim3(256), 0, stream, kp);
    else if (mode == 2) hipLaunchKernelGGL((k_bwd_main<DQK, DV, TM, 2, 0>), grid, dim3(256), 0, stream, kp);
    else hipLaunchKernelGGL((k_bwd_main<DQK, DV, TM, 0, 0>), grid, dim3(256), 0, stream, kp);
  }
}

hipError_t launch_main(const Plan& plan, const KParams& kp, hipStream_t stream) {
  const int64_t items = (int64_t)((plan.n_kv_tiles + plan.tiles_per_item - 1) / plan.tiles_per_item) *
                        plan.kv_parts * plan.Hkv * plan.B;
  if (items == 0) return hipSuccess;
  const dim3 grid((unsigned)items);
  if (plan.kernel == FMHA_KERNEL_WIDE) return launch_main_wide(plan, kp, grid, stream);
  if (plan.d_qk == 64) {
    if (plan.tile_m == 128) {
      launch_main_t<64, 64, 128, false>(plan, kp, grid, stream);  // bias: tile_m is 64
    } else {
      launch_main_t<64, 64, 64>(plan, kp, grid, stream);
    }
  } else if (plan.d_qk == 128) {
    if (plan.tile_m == 32) {
      launch_main_t<128, 128, 32>(plan, kp, grid, stream);
    } else {
      launch_main_t<128, 128, 64>(plan, kp, grid, stream);
    }
  } else {
    launch_main_t<192, 128, 32>(plan, kp, grid, stream);
  }
  return hipGetLastError();
}

template <int DQK, int TM>
static void launch_reduce_t(const Plan& plan, const KParams& kp, hipStream_t stream) {
  const int parts = plan.deterministic ? reduce_parts<DQK, TM>() : 1;
  const dim3 grid((unsigned)(plan.n_q_blocks * parts), (unsigned)plan.Hq, (unsigned)plan.B);
  hipLaunchKernelGGL((k_dq_reduce<DQK, TM>), grid, dim3(256), 0, stream, kp);
}

hipError_t launch_reduce(const Plan& plan, const KParams& kp, hipStream_t stream) {
  if (plan.n_q_blocks == 0 || plan.B == 0) return hipSuccess;
  if (plan.d_qk == 64) {
    if (plan.tile_m == 128) {
      launch_reduce_t<64, 128>(plan, kp, stream);
    } else if (plan.tile_m == 32) {
      launch_reduce_t<64, 32>(plan, kp, stream);  // the wide layout
    } else {
      launch_reduce_t<64, 64>(plan, kp, stream);
    }
  } else if (plan.d_qk == 128) {
    if (plan.tile_m == 32) {
      launch_reduce_t<128, 32>(plan, kp, stream);
    } else {
      launch_reduce_t<128, 64>(plan, kp, stream);
    }
  } else {
    launch_reduce_t<192, 32>(plan, kp, stream);
  }
  return hipGetLastError();
}

hipError_t launch_dkv_reduce(const Plan& plan, const KParams& kp, hipStream_t stream) {
  if (plan.kv_parts <= 1 || plan.B == 0 || plan.n_kv_tiles == 0) return hipSuccess;
  if (plan.kv_parts > 8) return hipErrorInvalidValue;  // the reduce sums at most 8 parts
  const dim3 grid((unsigned)(plan.n_kv_tiles * (plan.tile_n / kDkvRows)), (unsigned)plan.Hkv, (unsigned)plan.B);
  if (plan.d_qk == 64) {
    hipLaunchKernelGGL((k_dkv_reduce<64, 64>), grid, dim3(256), 0, stream, kp);
  } else if (plan.d_qk == 128) {
    hipLaunchKernelGGL((k_dkv_reduce<128, 128>), grid, dim3(256), 0, stream, kp);
  } else {
    hipLaunchKernelGGL((k_dkv_reduce<192, 128>), grid, dim3(256), 0, stream, kp);
  }
  return hipGetLastError();
}

hipError_t launch_dbias(const Plan& plan, const KParams& kp, hipStream_t stream) {
  if (!plan.has_dbias || plan.B == 0 || plan.Sq == 0 || plan.Sk == 0) return hipSuccess;
  const dim3 grid((unsigned)(((plan.Sk + 1023) / 1024) * (((int64_t)plan.Sq + kDbiasRows - 1) / kDbiasRows)),
                  (unsigned)plan.bias_h, (unsigned)plan.bias_b);
  hipLaunchKernelGGL(k_dbias_reduce, grid, dim3(256), 0, stream, kp);
  return hipGetLastError();
}

hipError_t launch_header(uint64_t* ws, uint64_t magic, uint64_t fingerprint, hipStream_t stream) {
  hipLaunchKernelGGL(k_header, dim3(1), dim3(64), 0, stream, ws, magic, fingerprint);
  return hipGetLastError();
}

hipError_t launch_zero_header(float* ptr, int64_t count, uint64_t* ws, uint64_t magic, uint64_t fingerprint,
                              hipStream_t stream) {
  const int64_t n4 = count / 4;  // the accumulator is a multiple of 4 floats (d_qk % 4 == 0)
  int64_t blocks = (n4 + 1023) / 1024;
  if (blocks < 1) blocks = 1;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(256), 0, stream, ptr, n4, ws, magic, fingerprint);
  return hipGetLastError();
}

}  // namespace fmha
