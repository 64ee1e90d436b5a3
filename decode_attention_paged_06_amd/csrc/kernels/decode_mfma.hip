// Paged decode attention on the gfx950 matrix cores.
//
// Operation: for one new query token per head, softmax(scale * q.K + alibi).V
// over the sequence's cached tokens, reached through its block table ("single
// query cached KV attention", vLLM PR #420; GQA head mapping of vLLM PR #452).
//
// Decomposition.  A workgroup owns the query heads that share one kv head (the
// GQA group, padded to NT tiles of 16 heads), for one sequence and one context
// partition -- or, under the equal-share schedule of the staged kernel (STREAM),
// for the pieces of (kv head, sequence) items that its equal share of the
// batch's tiles meets, one after the other.  A head tile is the N = 16 side of
// the MFMA products and each 16-row tile of cached tokens is the M = 16 side:
//
//   S^T[t, g]   = sum_d K[t, d] q[g, d]    v_mfma_f32_16x16x32_{f16,bf16}, D/32 steps
//   O^T[d, g]  += sum_t V[t, d] P[g, t]     v_mfma_f32_16x16x16_{f16,bf16}, D/16 tiles
//
// (multi-query calls, and staged decode over FP8 caches, take key tiles in
// pairs, KT = 2, and run P.V on the 16x16x32 form over the pair's 32 keys).
//
// The workgroup has NT x TG waves: wave w computes head tile w % NT (RT
// consecutive 16-row tiles of query rows for multi-query calls, which share
// each K/V operand and V regrouping) over the 16-row key tiles tg, tg + TG,
// tg + 2 TG, ... of the partition (tg = w / NT), with the K/V tiles ahead of
// the one being processed in flight: in registers (a software pipeline two
// tiles deep, three for FP8) when NT = 1, staged once per token group through
// an LDS ring when the NT tile-waves share every K/V tile.  The TG token groups' softmax states
// are merged at the end.
//
// Register layouts (lane = 16 j + r, r = lane % 16, j = lane / 16):
//   K operand, step i : lane holds K[t = r][8-element chunk c(i, j)], where
//                       c = 4i + j for 16-bit caches and 8(i/2) + 2j + i%2 for
//                       FP8 (one 16-byte read holds two steps); each read
//                       covers 64 contiguous bytes of each of the 16 rows.
//   q operand, step i : lane holds q[g = r][chunk c(i, j)]   (same k order as K).
//   scores            : lane holds S^T[t = 4j + v][g = r], v = 0..3.
//   V loads i = 0..3  : lane holds V[t = 4j + i][EPL elements at r * EPL]; each
//                       load reads 4 whole rows, fully coalesced.
//   P operand         : lane holds P[g = r][t = 4j + v]: exactly its scores,
//                       rounded to the storage type -- no data movement.
//   V^T operand, tile m: lane holds V[t = 4j + i][d = EPL r + m] for i = 0..3,
//                       regrouped from the four V loads with two v_perm_b32.
//   output tile m     : lane holds O^T[d = EPL (4j + v) + m][g = r], so lane
//                       (r, j) owns the contiguous output slice
//                       d in [4 EPL j, 4 EPL (j + 1)) of head r.
// The contraction index may be any permutation as long as both operands agree,
// which is what lines these layouts up with coalesced loads, with no
// re-layout of K or V on the way (a wave reading the LDS ring gets each
// lane's bytes as a direct load would have).
//
// Softmax: fp32 online softmax in log2 units against a reference max per
// head, shared by the 4 lane groups j (two lane swaps per step); each lane
// keeps a partial sum of its own rounded p values.  The reference moves (and
// l and the accumulators are rescaled) only when a step's max exceeds it by
// more than 8, so p stays below 2^8 and the rescale is rare.  P is rounded to
// the 16-bit compute type before the P.V product (the matrix cores take
// 16-bit operands); the sum l uses the same rounded values so the
// normalisation matches what was accumulated.
//
// FP8 caches: the tile is loaded as stored (1 byte per element, half the
// bytes) and converted exactly to the 16-bit compute format when processed;
// the key scale is folded into the logit scale and the value scale into the
// final normalisation, so the products above are unchanged.
#include <type_traits>

#include "../launch.h"
#include "device_common.h"

namespace pa {

template <typename Fmt>
struct Mfma;

template <>
struct Mfma<F16> {
  static __device__ __forceinline__ f32x4_t qk(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t pv(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t pv(uint4 a, uint4 b, f32x4_t c) {  // 32 keys
    return qk(a, b, c);
  }
};

template <>
struct Mfma<BF16> {
  static __device__ __forceinline__ f32x4_t qk(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t pv(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                     __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t pv(uint4 a, uint4 b, f32x4_t c) {  // 32 keys
    return qk(a, b, c);
  }
};

// EPL 16-bit elements per lane per V row load: 8 (uint4) for D = 128, 4 (uint2) for D = 64.
template <int EPL>
struct VRow;
template <>
struct VRow<8> {
  using T = uint4;
  static __device__ __forceinline__ uint32_t word(const T& v, int w) {
    return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
  }
};
template <>
struct VRow<4> {
  using T = uint2;
  static __device__ __forceinline__ uint32_t word(const T& v, int w) { return w == 0 ? v.x : v.y; }
};

template <typename Fmt, int D, int NT, int TG, int RT, int KT, bool KV8, bool STREAM = false>
__global__ __launch_bounds__(NT * TG * 64) void decode_mfma_kernel(const DecodeArgs a) {
  // Cache blocks of BS tokens are walked as tiles of TT = min(16, BS) rows, one
  // M = 16 MFMA tile each: a block of 32..256 tokens is BS/16 tiles sharing one
  // table lookup; an 8-token block is a half tile whose missing rows read back
  // as zeros from the bounds-checked buffer loads (and are masked).
  const int BS = a.block_size;
  const int TT = BS < 16 ? BS : 16;                                  // tokens per tile
  const int tpb_shift = a.block_shift > 4 ? a.block_shift - 4 : 0;  // log2(tiles per block)
  constexpr int CH = D / 8;     // 16-byte chunks per row
  constexpr int NK = D / 32;    // q.K MFMA steps
  constexpr int EPL = D / 16;   // V elements per lane per row load = number of P.V tiles
  using VR = VRow<EPL>;
  using VT = typename VR::T;
  using KS = KVStore<Fmt, KV8>;                  // cache storage (16-bit or FP8)
  constexpr int ES = KS::kBytes;                 // bytes per cached element
  using KRaw = typename KS::Raw8;                // 8 cached K elements (one q.K step)
  // K is read 16 bytes per lane: lane (r, j)'s read il covers row r, bytes
  // 16 j + 64 il .. + 16, and holds KSTEP q.K steps (dims are assigned to the
  // steps in that order; the query operand uses the same assignment).  Each
  // read instruction thus covers 64 contiguous bytes of each of 16 rows.
  constexpr int KSTEP = KS::kKSteps;
  constexpr int NKL = NK / KSTEP;                // K reads per tile
  using VRaw = typename std::conditional<EPL == 8, typename KS::Raw8, typename KS::Raw4>::type;
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr float kRescaleSlack = 8.f;  // log2 units: weights stay below 256
  // register tiles in the load pipeline (one wave per tile); FP8 tiles are half
  // the size, and a third one in flight measured ~1% faster
  constexpr int kDepth = KV8 ? 3 : 2;
  // With several head tiles the NT waves of a token group need the same K/V
  // tile: it is staged once through a ring of kRing LDS slots instead.
  constexpr bool STAGE = NT > 1;
  // KT = 2: the LDS ring holds pairs of consecutive tiles, processed together
  // (one softmax max per 32 keys; P.V on the 32-deep MFMA, whose two operands
  // are the two tiles' 16-key operands side by side); multi-query calls and
  // staged decode over FP8 caches
  static_assert(KT == 1 || (KT == 2 && STAGE), "tile pairs are staged");
  constexpr int kRing = KT == 2 ? 3 : 4;  // ring slots (of KT tiles)
  // A staged tile: K as per-lane 16-byte pieces, V as the tile's own 16 rows
  // (contiguous in the cache), read back at the direct-load offsets (TRV:
  // K, like V, as the tile's 16 rows with swizzled pieces; see below).
  //
  // TRV (staged, 16-bit caches, D = 128): the P.V operand V^T is read from
  // the ring with LDS transpose reads instead of being regrouped in
  // registers.  A transpose read hands lane i of each 16-lane group element
  // i % 4 of the 8-byte pieces that lanes i / 4 + 4 k (k = 0..3) point at, so
  // with lane (group g, k, q) pointing at V row 4 g + k, dims 16 m + 4 q ..,
  // lane (r, g) receives V[4 g + k][16 m + r], k = 0..3: the operand of
  // output tile m (16 consecutive dims).  Rows are 256 bytes, so the 16-byte
  // pieces of row t are stored XOR-swizzled by 2 t (piece p at p ^ 2 t mod
  // 16): a read's lanes want pieces 2 m and 2 m + 1 of 4 (per 128 bytes the
  // LDS serves) or 8 (per 256) consecutive rows, and those land on distinct
  // 8-byte bank slots, so no read waits on a bank conflict.
  constexpr bool TRV = STAGE && !KV8 && D == 128;
  using KPiece = LdsPiece;
  constexpr int kVBytes = 16 * D * ES;
  constexpr int kStageBytes = NKL * KPiece::kBytes + kVBytes;
  constexpr int kRingBytes = STAGE ? TG * kRing * KT * kStageBytes : 0;
  constexpr int ROWS = NT * RT * 16;  // query rows per workgroup (RT 16-row tiles per wave)
  // token groups 1 .. TG - 1 each leave their softmax state in a slot
  constexpr int kMergeSlotBytes = NT * RT * (EPL * 64 * 16 + 2 * 64 * 4);
  constexpr int kMergeBytes = TG > 1 ? (TG - 1) * kMergeSlotBytes : 0;
  constexpr int kQueryBytes = ROWS * (D / 8) * 16;
  constexpr int kWorkBytes0 = kRingBytes > kMergeBytes ? kRingBytes : kMergeBytes;
  constexpr int kWorkBytes = kWorkBytes0 > kQueryBytes ? kWorkBytes0 : kQueryBytes;
  // the query rows before the tile loop (they move to registers first), the
  // ring during it, the token-group merge after it
  __shared__ __align__(16) char work_lds[kWorkBytes];
  constexpr int kTableWindow = 512;  // tile source offsets held in LDS by the staged loop
  __shared__ uint64_t toff_lds[STAGE ? kTableWindow : 1];
  using Lds = DecodeLds<D, NT, TG, RT, KT, KV8>;
  static_assert(Lds::kStageBytes == kStageBytes && Lds::kRing == kRing && Lds::kWorkBytes == kWorkBytes &&
                    Lds::kTableWindow == kTableWindow,
                "DecodeLds describes this kernel's LDS");

  constexpr int NTHREADS = NT * TG * 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int tile = wave % NT;  // head tile of this wave
  const int tg = wave / NT;    // token group of this wave
  const int r = lane & 15;
  const int j = lane >> 4;

  // ---- the work ---------------------------------------------------------------
  // Grid schedules: one unit (row chunk, kv head, sequence, partition) per
  // workgroup.  Equal shares (decode on the staged kernel, stream_wgs > 0):
  // the batch's tiles, walked item by item (item = kv head * num_seqs +
  // sequence), are cut into consecutive shares of equal cost (tiles plus a
  // fixed cost per item; below), one per workgroup, and the workgroup
  // processes the pieces of the items its share meets, one after the other
  // (pieces of one item from several workgroups meet in the reduce).
  // A unit (piece): rows of row chunk / kv head xi of sequence seq, tiles
  // t_lo .. t_hi - 1 of the sequence (tiles of TT tokens).
  constexpr bool stream = STREAM;
  static_assert(!STREAM || STAGE, "equal shares run on the staged kernel");
  static_assert(!STREAM || (kStreamMaxSeqs + 1) * 4 <= kWorkBytes, "the tile prefix fits the work area");
  auto unit = [&](int xi, int seq, int part, int t_lo, int t_hi, int item) {
    // ---- which query rows this workgroup owns ---------------------------------
    // A row is a (new token i, query head g) pair of one sequence and kv head,
    // numbered i * G + g; the workgroup owns ROWS consecutive rows, RT tiles of
    // 16 per wave.  Decode has one new token per sequence, so its rows are the
    // group's G heads.
    if (stream) __syncthreads();  // the previous piece's LDS (and the tile prefix) are free
    const int chunks = a.row_chunks;
    // kv heads vary fastest, and row chunks run from the last one down: with
    // multi-query rows a later chunk sees more keys (its rows sit later in the
    // sequence), so the longest work units start first (measured +13..24% on
    // causal multi-query batches against the ascending order)
    const int kvh = xi % a.num_kv_heads;
    const int rc = chunks - 1 - xi / a.num_kv_heads;
    const int G = a.group;
    const int h0 = kvh * G;
    const bool single = !stream && a.num_partitions == 1;
    int q_first = seq, n_new = 1;  // packed index of the sequence's first new token
    if (a.query_start != nullptr) {
      q_first = a.query_start[seq];
      n_new = a.query_start[seq + 1] - q_first;
    }
    const int row_base = rc * ROWS;
    const int nrows = n_new * G;
    if (row_base >= nrows) return;  // this sequence has fewer rows

    // The query rows, and the block ids of this wave's first two tiles (their
    // table positions do not depend on the context length), are requested
    // before the context length is known, so the three loads overlap.
    const int* table = a.block_tables + (size_t)seq * a.max_blocks_per_seq;
    const int tile0 = t_lo;  // first tile of the partition (piece)
    auto block_at = [&](int u) {  // table entry of tile u (clamped to the table)
      return table[min((tile0 + u) >> tpb_shift, a.max_blocks_per_seq - 1)];
    };
    const int ctx_len = a.context_lens[seq];
    int blk_first = 0, blk_second = 0;
    if constexpr (!STAGE) {
      blk_first = block_at(tg);
      blk_second = block_at(tg + TG);
    }
    // ---- shared query load: the owned rows, zero-padded to ROWS -------------
    uint4* q_lds = reinterpret_cast<uint4*>(work_lds);
    for (int idx = threadIdx.x; idx < ROWS * CH; idx += NTHREADS) {
      const int rr = row_base + idx / CH;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (rr < nrows) {
        const int ti = rr / G;
        v = reinterpret_cast<const uint4*>(a.q)[((size_t)(q_first + ti) * a.num_heads + h0 + rr - ti * G) *
                                                    CH + idx % CH];
      }
      q_lds[idx] = v;
    }
    asm volatile("" ::"s"(ctx_len));  // its load was in flight with the query's
    __syncthreads();
    const int L = min(ctx_len, a.max_blocks_per_seq * BS);
    if (L <= 0) {
      if (single) {  // no context: zero output rows
        for (int idx = threadIdx.x; idx < ROWS * CH; idx += NTHREADS) {
          const int rr = row_base + idx / CH;
          if (rr < nrows) {
            const int ti = rr / G;
            reinterpret_cast<uint4*>(a.out)[((size_t)(q_first + ti) * a.num_heads + h0 + rr - ti * G) * CH +
                                            idx % CH] = make_uint4(0, 0, 0, 0);
          }
        }
      }
      return;
    }
    // the owned rows see keys up to the position of the last owned new token
    const int last_new = min(n_new, (row_base + ROWS + G - 1) / G) - 1;
    const int kend = L - n_new + last_new + 1;
    const int tok0 = t_lo * TT;
    if (tok0 >= kend) return;  // partition past every owned row's keys: nothing to do
    const int tok1 = min(kend, t_hi * TT);
    // (equal shares) the piece is the whole item: the reduce leaves its rows alone
    const bool whole = stream && t_lo == 0 && tok1 == kend;
    const int ntiles = (tok1 - tok0 + TT - 1) / TT;  // tiles holding its tokens

    // This lane's rows: row r of each of the wave's RT row tiles.
    bool row_ok[RT];
    int ti[RT], g[RT], pos[RT], pos_lo[RT];
    uint4 qb[RT][NK];
    float slope[RT];
    const bool has_alibi = a.alibi != nullptr;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int rt_base = row_base + (tile * RT + rt) * 16;
      const int row = rt_base + r;
      row_ok[rt] = row < nrows;
      ti[rt] = row / G;             // its new token
      g[rt] = row - ti[rt] * G;     // its query head within the group
      // its position: keys 0 .. pos are visible (padding rows, past the last
      // new token, get a position past L; their results are never stored)
      pos[rt] = L - n_new + ti[rt];
      // the lowest position among the tile's 16 rows (wave-uniform): key tiles
      // that end at or before it, and are full, need no masking
      pos_lo[rt] = L - n_new + rt_base / G;
#pragma unroll
      for (int i = 0; i < NK; ++i)
        qb[rt][i] = q_lds[((tile * RT + rt) * 16 + r) * CH + (i / KSTEP) * 4 * KSTEP + j * KSTEP + i % KSTEP];
      slope[rt] = (has_alibi && row_ok[rt]) ? a.alibi[h0 + g[rt]] * kLog2e : 0.f;
      // the slope's load completes here, before the tile loop's own memory traffic
      asm volatile("" ::"v"(slope[rt]));
    }

    float m[RT], lsum[RT];
    f32x4_t acc[RT][EPL];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      m[rt] = kNegBig;
      lsum[rt] = 0.f;
#pragma unroll
      for (int t = 0; t < EPL; ++t) acc[rt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // Byte addressing: a wave-uniform tile base (SGPRs) plus a small unsigned
    // per-lane offset, so every K/V load is one buffer load with a VGPR offset.
    const size_t bstride = (size_t)a.kv_block_stride;  // bytes per physical block
    const size_t head_off = (size_t)kvh * (size_t)a.kv_head_stride;
    const char* kbase = reinterpret_cast<const char*>(a.k_cache) + head_off;
    const char* vbase = reinterpret_cast<const char*>(a.v_cache) + head_off;
    const uint32_t k_lane = (uint32_t)(r * D * ES + j * 16);         // read-0 K chunk
    const uint32_t v_lane = (uint32_t)((4 * j) * D + r * EPL) * ES;  // load-0 V slice
    // TRV: the K and V source offsets of this lane in LDS transfer c (rows
    // 4 c .. 4 c + 3; the transfer's own 1 KB step comes from its immediate
    // offset), the K read offset of q.K step i and the transpose-read offset of
    // output tile m in a staged tile.  Staged K rows keep their 16-byte pieces
    // XOR-swizzled by the row index (piece p at p ^ t): a K read's lanes (rows
    // r, pieces 4 i + j) then never share a bank, and the tile's K takes one
    // M0 set-up and four transfers like its V.
    uint32_t v_swz[TRV ? 4 : 1], v_tr[TRV ? 8 : 1], k_swz[TRV ? 4 : 1], k_rd[TRV ? 4 : 1];
    if constexpr (TRV) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        k_swz[c] = (uint32_t)(j * 256 + ((r ^ (4 * c + j)) & 15) * 16);
        k_rd[c] = (uint32_t)(r * 256 + (((4 * c + j) ^ r) & 15) * 16);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
        v_swz[c] = (uint32_t)(j * 256 + ((r ^ (2 * (4 * c + j))) & 15) * 16);
      const int row = 4 * j + (r >> 2), q = r & 3;
#pragma unroll
      for (int m = 0; m < 8; ++m)
        v_tr[m] = (uint32_t)(row * 256 + (((2 * m + (q >> 1)) ^ (2 * row)) & 15) * 16 + (q & 1) * 8);
    }

    // One 16-row tile's K and V in registers, as stored in the cache.
    struct Tile {
      KRaw k[NK];
      VRaw v[4];
    };
    // u: tile index within the partition; blk: its physical block (the table
    // entry is read one tile ahead of the load that needs it, so the scalar
    // load's latency hides behind a tile's processing).  The buffer bound is
    // the tile's valid rows: rows past the context end (which may hold
    // anything, NaN included) read back as zeros, and a tile past the end of
    // the partition (u >= ntiles) reads nothing at all.  Every pipeline step
    // thus issues the same loads, which keeps the wait counts exact.
    auto block_of = [&](int u) { return block_at(min(u, ntiles - 1)); };
    auto load = [&](Tile& T, int u, int blk) {
      const int ua = tile0 + u;
      const size_t off = (size_t)blk * bstride + (size_t)(ua & ((1 << tpb_shift) - 1)) * (16 * D * ES);
      const uint32_t bytes = u < ntiles ? (uint32_t)min(tok1 - ua * TT, TT) * (D * ES) : 0u;
      const rsrc_t rk = make_rsrc(kbase + off, bytes);
      const rsrc_t rv = make_rsrc(vbase + off, bytes);
#pragma unroll
      for (int i = 0; i < NKL; ++i)
        KS::split(buffer_load<NT == 1>(rk, k_lane + 64u * i, (uint4*)nullptr), &T.k[i * KSTEP]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (EPL == 8) T.v[i] = KS::template load8<NT == 1>(rv, v_lane + (uint32_t)D * ES * i);
        else T.v[i] = KS::template load4<NT == 1>(rv, v_lane + (uint32_t)D * ES * i);
      }
    };

    // T: KT consecutive tiles u0, u0 + 1, ...; vlds (TRV): their staged V
    // tiles, kStageBytes apart
    auto process = [&](const Tile* T, int u0, const char* vlds) {
      // the compute format of the tiles (a no-op for 16-bit caches)
      uint4 kk[KT][NK];
      VT vv[KT][4];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int i = 0; i < NK; ++i) kk[kt][i] = KS::to16(T[kt].k[i]);
        if constexpr (!TRV) {
#pragma unroll
          for (int i = 0; i < 4; ++i) vv[kt][i] = KS::to16(T[kt].v[i]);
        }
      }

      // scores and weights of each row tile (the K tiles are shared)
      using PK = typename std::conditional<KT == 2, uint4, uint2>::type;
      PK pk[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        // x: a tile's logits in log2 units, or (full tile, no ALiBi, positive
        // scale) its raw scores, with the scale applied in the exponent below;
        // xs is what x is multiplied by to get the logit
        float x[KT][4], xs[KT];
        float local = kNegBig;  // this lane's largest logit
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const int tb = (tile0 + u0 + kt) * TT;  // absolute position of the tile's row 0
          const int valid = min(tok1 - tb, TT);   // rows [0, valid) are context tokens
          f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < NK; ++i) sc = Mfma<Fmt>::qk(kk[kt][i], qb[rt][i], sc);
          xs[kt] = 1.f;
          if (valid == 16 && tb + 15 <= pos_lo[rt]) {  // every row sees every key of the tile
            if (has_alibi) {
              const float base = slope[rt] * (float)(tb + 4 * j - pos[rt]);
#pragma unroll
              for (int v = 0; v < 4; ++v)
                x[kt][v] = fmaf(sc[v], a.scale_log2, fmaf((float)v, slope[rt], base));
            } else if (a.scale_log2 > 0.f) {
#pragma unroll
              for (int v = 0; v < 4; ++v) x[kt][v] = sc[v];
              xs[kt] = a.scale_log2;
            } else {
#pragma unroll
              for (int v = 0; v < 4; ++v) x[kt][v] = sc[v] * a.scale_log2;
            }
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int t = 4 * j + v;
              const float z = fmaf(sc[v], a.scale_log2, slope[rt] * (float)(tb + t - pos[rt]));
              x[kt][v] = (t < valid && tb + t <= pos[rt]) ? z : kNegBig;
            }
          }
          local = score_max(local, xs[kt] * score_max(score_max(x[kt][0], x[kt][1]),
                                                       score_max(x[kt][2], x[kt][3])));
        }
        // The reference max m moves only when some row's max over the step
        // exceeds it by more than kRescaleSlack (weights then stay below
        // 2^kRescaleSlack): the rescale of l and the accumulators is rare, and
        // the result is the same quotient acc / l whichever m it is taken against.
        // Each lane tests its own keys; only a step that moves m takes the row
        // max across the four lane groups, so all four move m alike.
        if (wave_any(local > m[rt] + kRescaleSlack)) {
          const float mn = score_max(m[rt], column_max4(local));
          const float alpha = fast_exp2(m[rt] - mn);
          m[rt] = mn;
          lsum[rt] *= alpha;
#pragma unroll
          for (int t = 0; t < EPL; ++t) acc[rt][t] *= alpha;
        }
        const float nm = -m[rt];
        uint32_t pw[2 * KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          pw[2 * kt] = Fmt::pack(fast_exp2(fmaf(x[kt][0], xs[kt], nm)), fast_exp2(fmaf(x[kt][1], xs[kt], nm)));
          pw[2 * kt + 1] =
              Fmt::pack(fast_exp2(fmaf(x[kt][2], xs[kt], nm)), fast_exp2(fmaf(x[kt][3], xs[kt], nm)));
          // l sums the rounded weights that P.V uses (products by one are exact)
          lsum[rt] = Fmt::dot2(pw[2 * kt + 1], Fmt::kOnes, Fmt::dot2(pw[2 * kt], Fmt::kOnes, lsum[rt]));
        }
        if constexpr (KT == 2) pk[rt] = make_uint4(pw[0], pw[1], pw[2], pw[3]);
        else pk[rt] = make_uint2(pw[0], pw[1]);
      }

      // P.V: the V^T operand of each output tile is regrouped once and serves
      // every row tile; with tile pairs the contraction runs over 32 keys, the
      // first tile's 4 keys of each lane group followed by the second's (the
      // weights above are laid out the same way)
#pragma unroll
      for (int t = 0; t < EPL; ++t) {
        uint2 vt[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          if constexpr (TRV) {
            typedef short v4s_t __attribute__((ext_vector_type(4)));
            typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;
            const v4s_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4s_t*)(lds_void_t*)(vlds + kt * kStageBytes + v_tr[t]));
            vt[kt] = __builtin_bit_cast(uint2, x);
          } else {
            const int w = t >> 1;
            const uint32_t a0 = VR::word(vv[kt][0], w), a1 = VR::word(vv[kt][1], w);
            const uint32_t a2 = VR::word(vv[kt][2], w), a3 = VR::word(vv[kt][3], w);
            vt[kt] = (t & 1) ? make_uint2(pack_hi_hi(a0, a1), pack_hi_hi(a2, a3))
                             : make_uint2(pack_lo_lo(a0, a1), pack_lo_lo(a2, a3));
          }
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          if constexpr (KT == 2)
            acc[rt][t] = Mfma<Fmt>::pv(make_uint4(vt[0].x, vt[0].y, vt[1].x, vt[1].y), pk[rt], acc[rt][t]);
          else
            acc[rt][t] = Mfma<Fmt>::pv(vt[0], pk[rt], acc[rt][t]);
        }
      }
    };

    if constexpr (!STAGE) {
      // Software pipeline of kDepth register tiles used in rotation: while one
      // tile is processed, the loads of the wave's next kDepth - 1 tiles are in
      // flight.
      Tile buf[kDepth];
      int u = tg;
      if (u < ntiles) {
        // the first two block ids were fetched with the query
        const int blk_1 = u + TG < ntiles ? blk_second : blk_first;
        load(buf[0], u, blk_first);
#pragma unroll
        for (int k = 1; k + 1 < kDepth; ++k) load(buf[k], u + k * TG, k == 1 ? blk_1 : block_of(u + k * TG));
        int blk_next = kDepth == 2 ? blk_1 : block_of(u + (kDepth - 1) * TG);
        bool more = true;
        while (more) {
#pragma unroll
          for (int k = 0; k < kDepth; ++k) {
            if (more) {
              const int uc = u + k * TG;
              load(buf[(k + kDepth - 1) % kDepth], uc + (kDepth - 1) * TG, blk_next);
              blk_next = block_of(uc + kDepth * TG);
              process(&buf[k], uc, nullptr);
              more = uc + TG < ntiles;
            }
          }
          u += kDepth * TG;
        }
      }
    } else {
      // LDS ring: the first wave of each token group copies tile tg + j TG into
      // slot j % kRing, kRing - 1 tiles ahead; after its wait and a barrier
      // every wave of the group reads the tile from the slot (splitting the
      // copy between two waves, K and V, measured no faster).  All waves of the workgroup run the same number of steps
      // (every step has a barrier); a group's steps past its last tile copy
      // nothing and process nothing.
      //
      // Source offsets of the partition's tiles (block-table entry times the
      // block stride, plus the tile's place in its block) come from a window of
      // kTableWindow tiles kept in LDS: the table lookup and the 64-bit product
      // are done once per tile, by all lanes, when the window is filled, and a
      // step's copy only adds its base.  Entries past the last tile repeat it
      // (their copies read nothing).  The copies write memory the compiler
      // cannot tell apart from the table, so the table is not read with scalar
      // loads inside the loop.  The window is refilled by all waves, between
      // barriers, when the tiles being copied move past it.
      const uint64_t bstride64 = (uint64_t)a.kv_block_stride;
      const int tpb_mask = (1 << tpb_shift) - 1;
      auto fill_window = [&](int start) {
        for (int i = threadIdx.x; i < kTableWindow; i += NTHREADS) {
          const int ua = tile0 + min(start + i, ntiles - 1);
          toff_lds[i] = (uint64_t)(uint32_t)table[ua >> tpb_shift] * bstride64 +
                        (uint32_t)((ua & tpb_mask) * (16 * D * ES));
        }
      };
      int win0 = 0;  // first tile of the window
      fill_window(0);
      __syncthreads();

      char* ring = work_lds + tg * (kRing * KT * kStageBytes);
      const bool copier = tile == 0;
      constexpr int kCopyTransfers = NKL * KPiece::kTransfers + kVBytes / 1024;  // per tile
      // ring slots hold KT consecutive tiles: step unit us covers tiles
      // us KT .. us KT + KT - 1 (those past the partition read nothing).
      // The copier reads the next step's offsets right after its copy (their LDS
      // round trip then hides behind the step), except across a window refill.
      // An offset outside the window is clamped into it and only ever used for
      // a step that refills first (and reads its offsets again).
      auto window_offs = [&](int us, uint64_t* o) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
          o[kt] = toff_lds[min(min(us * KT + kt, ntiles - 1) - win0, kTableWindow - 1)];
      };
      auto copy = [&](int us, int slot, const uint64_t* offs) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const int u = us * KT + kt;
          const int ua = tile0 + u;
          const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)offs[kt]);
          const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(offs[kt] >> 32));
          const uint64_t off = ((uint64_t)hi << 32) | lo;
          const uint32_t bytes = u < ntiles ? (uint32_t)min(tok1 - ua * TT, TT) * (D * ES) : 0u;
          char* dst = ring + (slot * KT + kt) * kStageBytes;
          const rsrc_t rk = make_rsrc(kbase + off, bytes);
          const rsrc_t rv = make_rsrc(vbase + off, bytes);
          if constexpr (TRV) {
            lds_copy_rows_swizzled(rk, dst, k_swz);
          } else {
#pragma unroll
            for (int i = 0; i < NKL; ++i) KPiece::copy(rk, k_lane + 64u * i, dst + i * KPiece::kBytes);
          }
          if constexpr (TRV) lds_copy_rows_swizzled(rv, dst + NKL * KPiece::kBytes, v_swz);
          else lds_copy_run<kVBytes>(rv, dst + NKL * KPiece::kBytes, lane);
        }
      };
      auto read = [&](Tile& T, int slot, int kt) {
        const char* src = ring + (slot * KT + kt) * kStageBytes;
#pragma unroll
        for (int i = 0; i < NKL; ++i) {
          if constexpr (TRV) KS::split(*reinterpret_cast<const uint4*>(src + k_rd[i]), &T.k[i * KSTEP]);
          else KS::split(KPiece::read(src + i * KPiece::kBytes, lane), &T.k[i * KSTEP]);
        }
        if constexpr (!TRV) {  // (TRV: P.V reads V itself, transposed)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            T.v[i] = *reinterpret_cast<const VRaw*>(src + NKL * KPiece::kBytes + v_lane + (uint32_t)D * ES * i);
        }
      };
      const int nunits = (ntiles + KT - 1) / KT;
      const int nsteps = (nunits + TG - 1) / TG;
      uint64_t offs[KT];
      // Decode walks the partition's units last to first when the window holds
      // all of them: with ALiBi the bias grows toward the query token, so the
      // running max is set by the first units and the rescale of the
      // accumulators (every unit, for the steep slopes, in ascending order) is
      // rare (MQA 48/1 ALiBi batch 256, FP8 cache: 93.3 -> 86.8 us; 16-bit
      // 104.6 -> 103.9 us).  Every unit of a decode partition holds a key the
      // row sees, so the first unit sets a finite max.  Multi-query rows can
      // see none of a late unit's keys, so they keep the ascending order.
      const bool reverse = a.query_start == nullptr && ntiles <= kTableWindow;
      auto order = [&](int u) { return reverse && u < nunits ? nunits - 1 - u : u; };
      if (copier) {
#pragma unroll
        for (int k = 0; k + 1 < kRing; ++k) {
          window_offs(order(tg + k * TG), offs);
          copy(order(tg + k * TG), k, offs);
        }
        window_offs(order(tg + (kRing - 1) * TG), offs);  // step 0's
      }
      // One step; its ring slot is a compile-time constant (the loop below is
      // unrolled by the ring size), so every LDS address of the tile reads is a
      // loop-invariant lane offset plus an immediate (MQA 48/1: one address add
      // fewer per K and V^T read).
      auto step = [&](int j, auto slot_tag) {
        constexpr int kSlot = decltype(slot_tag)::value;  // j % kRing
        if (copier) wait_vmcnt<kCopyTransfers * KT * (kRing - 2)>();  // unit j has landed
        // the units copied in this step are (j + kRing - 1) TG + 0 .. TG - 1
        const int first = (j + kRing - 1) * TG;
        const bool refill = min((first + TG) * KT, ntiles) - 1 - win0 >= kTableWindow;  // same for every wave
        if (refill) {
          lds_barrier();  // every copier is done with the old window
          win0 = first * KT;
          fill_window(win0);
          asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        }
        lds_barrier();  // unit j is visible to every wave; slot (j - 1) % kRing is free
        if (copier) {
          if (refill) window_offs(order(tg + first), offs);
          copy(order(tg + first), (kSlot + kRing - 1) % kRing, offs);
          window_offs(order(tg + first + TG), offs);  // the next step's
        }
        const int uc = tg + j * TG;
        if (uc < nunits) {
          Tile T[KT];
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) read(T[kt], kSlot, kt);
          process(T, order(uc) * KT, ring + kSlot * KT * kStageBytes + NKL * KPiece::kBytes);
        }
      };
      static_assert(kRing == 3 || kRing == 4, "the loop is unrolled by the ring size");
      for (int j = 0; j < nsteps; j += kRing) {
        step(j, std::integral_constant<int, 0>{});
        if (j + 1 < nsteps) step(j + 1, std::integral_constant<int, 1>{});
        if (j + 2 < nsteps) step(j + 2, std::integral_constant<int, 2>{});
        if constexpr (kRing == 4) {
          if (j + 3 < nsteps) step(j + 3, std::integral_constant<int, kRing == 4 ? 3 : 0>{});
        }
      }
      if (copier) wait_vmcnt<0>();  // the copies past the end have landed before the LDS is reused
    }

    // ---- complete the per-lane sums over the 4 lane groups -------------------
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) lsum[rt] = column_sum4(lsum[rt]);

    // ---- merge the token groups into group 0 (fixed order: deterministic) ----
    // Groups 1 .. TG - 1 write their states to their own slots at once; after
    // a barrier group 0 folds them in, in group order (two barriers in all
    // rather than two per group).
    if constexpr (TG > 1) {
      __syncthreads();  // every wave is past its reads of the query / the ring, which the slots reuse
      auto slot_base = [&](int k) { return work_lds + (k - 1) * kMergeSlotBytes; };
      if (tg != 0) {
        char* base = slot_base(tg);
        auto mrg_acc = reinterpret_cast<f32x4_t(*)[EPL][64]>(base);
        auto mrg_m = reinterpret_cast<float(*)[64]>(base + NT * RT * EPL * 64 * 16);
        auto mrg_l = reinterpret_cast<float(*)[64]>(base + NT * RT * EPL * 64 * 16 + NT * RT * 64 * 4);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int slot = tile * RT + rt;
          mrg_m[slot][lane] = m[rt];
          mrg_l[slot][lane] = lsum[rt];
#pragma unroll
          for (int t = 0; t < EPL; ++t) mrg_acc[slot][t][lane] = acc[rt][t];
        }
      }
      __syncthreads();
      if (tg == 0) {
        for (int k = 1; k < TG; ++k) {
          const char* base = slot_base(k);
          auto mrg_acc = reinterpret_cast<const f32x4_t(*)[EPL][64]>(base);
          auto mrg_m = reinterpret_cast<const float(*)[64]>(base + NT * RT * EPL * 64 * 16);
          auto mrg_l = reinterpret_cast<const float(*)[64]>(base + NT * RT * EPL * 64 * 16 + NT * RT * 64 * 4);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const int slot = tile * RT + rt;
            const float mo = mrg_m[slot][lane];
            const float mn = score_max(m[rt], mo);
            const float f = fast_exp2(m[rt] - mn);
            const float fo = fast_exp2(mo - mn);
            lsum[rt] = lsum[rt] * f + mrg_l[slot][lane] * fo;
#pragma unroll
            for (int t = 0; t < EPL; ++t) acc[rt][t] = acc[rt][t] * f + mrg_acc[slot][t][lane] * fo;
            m[rt] = mn;
          }
        }
      }
    }

    // ---- finalise ---------------------------------------------------------------
    // A row whose visible keys (0 .. pos) all lie in partition 0, or (equal
    // shares) whose item this workgroup holds whole, is finished here; the
    // reduce skips it.
    if (tg != 0) return;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if (!row_ok[rt]) continue;
      const float inv = lsum[rt] > 0.f ? a.v_scale / lsum[rt] : 0.f;
      const size_t orow_idx = (size_t)(q_first + ti[rt]) * a.num_heads + h0 + g[rt];
      if (stream ? whole : single || (part == 0 && pos[rt] < a.partition_blocks * BS)) {
        uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + orow_idx * D;
        if constexpr (TRV) {  // output tile t: dims 16 t + 4 j .. + 3 of head r
#pragma unroll
          for (int t = 0; t < EPL; ++t)
            *reinterpret_cast<uint2*>(orow + 16 * t + 4 * j) =
                make_uint2(Fmt::pack(acc[rt][t][0] * inv, acc[rt][t][1] * inv),
                           Fmt::pack(acc[rt][t][2] * inv, acc[rt][t][3] * inv));
        } else {  // output tiles: dims EPL (4 j + v) + t of head r
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            uint32_t wv[EPL / 2];
#pragma unroll
            for (int t = 0; t < EPL; t += 2)
              wv[t / 2] = Fmt::pack(acc[rt][t][v] * inv, acc[rt][t + 1][v] * inv);
            VT o;
            if constexpr (EPL == 8) o = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            else o = make_uint2(wv[0], wv[1]);
            *reinterpret_cast<VT*>(orow + EPL * (4 * j + v)) = o;
          }
        }
      } else {
        const size_t slot = stream ? (size_t)g[rt] * a.num_slots + item + blockIdx.x
                                   : orow_idx * a.num_partitions + part;
        float* orow = a.ws_o + slot * D;
        if constexpr (TRV) {
#pragma unroll
          for (int t = 0; t < EPL; ++t)
            *reinterpret_cast<float4*>(orow + 16 * t + 4 * j) =
                make_float4(acc[rt][t][0] * inv, acc[rt][t][1] * inv, acc[rt][t][2] * inv, acc[rt][t][3] * inv);
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
#pragma unroll
            for (int t = 0; t < EPL; t += 4)
              *reinterpret_cast<float4*>(orow + EPL * (4 * j + v) + t) =
                  make_float4(acc[rt][t][v] * inv, acc[rt][t + 1][v] * inv, acc[rt][t + 2][v] * inv,
                              acc[rt][t + 3][v] * inv);
          }
        }
        if (j == 0) reinterpret_cast<float2*>(a.ws_ml)[slot] = make_float2(m[rt], lsum[rt]);
      }
    }

  };

  // Equal shares.  A kv head's stream is its sequences in order, each as
  // piece_cost positions that stand for a piece's fixed start-up and finish
  // (query and table loads, token-group merge, partial store) followed by one
  // position per tile; workgroup b takes positions [floor(b T / G),
  // floor((b + 1) T / G)) of the kv heads' streams laid end to end and
  // processes the tiles among them, item by item.  Wave 0 builds each
  // sequence's first tile (the exclusive prefix of ceil(L / TT)) in LDS, 512
  // sequences a pass, then finds the sequence where the share starts.
  const int S = a.num_seqs;
  const int nitems = stream ? S * a.num_kv_heads : 1;
  const int64_t cost = a.piece_cost;
  const int maxlen = a.max_blocks_per_seq * BS;
  int it_first = 0;
  int64_t X0 = 0, X1 = 0, C = 0;  // the share [X0, X1); C: where the current item's positions start
  if (stream) {
    int* pfx = reinterpret_cast<int*>(work_lds);
    int* found = reinterpret_cast<int*>(toff_lds);  // (filled with tile offsets only later)
    if (wave == 0) {
      int carry = 0;
      for (int c = 0; c < S; c += 512) {
        int v[8], tot = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int sq = c + lane * 8 + k;
          const int L = sq < S ? min(a.context_lens[sq], maxlen) : 0;
          v[k] = L > 0 ? (L + TT - 1) / TT : 0;
          tot += v[k];
        }
        const int incl = wave_prefix_sum(tot);
        int run = carry + incl - tot;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int sq = c + lane * 8 + k;
          if (sq < S) pfx[sq] = run;
          run += v[k];
        }
        carry += __shfl(incl, 63, 64);
      }
      if (lane == 0) pfx[S] = carry;
    }
    __syncthreads();
    const int64_t T1 = pfx[S] + cost * S;   // positions of one kv head
    const int64_t T = T1 * a.num_kv_heads;  // stream length
    // shares of at least one position each (the reduce counts the same way)
    const int64_t nwg = T < (int64_t)gridDim.x ? T : (int64_t)gridDim.x;
    X0 = stream_share_start(blockIdx.x, T, nwg);
    X1 = stream_share_start(blockIdx.x + 1, T, nwg);
    it_first = nitems;
    if (X0 < T) {  // the sequence s whose positions [pfx[s] + cost s, pfx[s + 1] + cost (s + 1)) hold X0
      const int kv = (int)(X0 / T1);
      const int64_t o = X0 - kv * T1;
      if (wave == 0)
        for (int sq = lane; sq < S; sq += 64)
          if (pfx[sq] + cost * sq <= o && o < pfx[sq + 1] + cost * (sq + 1)) found[0] = sq;
      __syncthreads();
      const int s0 = __builtin_amdgcn_readfirstlane(found[0]);
      it_first = kv * S + s0;
      C = kv * T1 + pfx[s0] + cost * s0;
    }
    if (blockIdx.x == 0)  // the prefix, for the reduce
      for (int i = threadIdx.x; i <= S; i += NTHREADS) a.ws_pfx[i] = pfx[i];
  }
  // (equal shares) the next item's context length, requested an item ahead
  int len_next = stream && it_first < nitems ? a.context_lens[it_first % S] : 0;
  for (int it = it_first; stream ? it < nitems && C < X1 : it < 1; ++it) {
    int xi, seq, part, t_lo, t_hi;
    if (stream) {  // the piece of item it in the share
      xi = it / S;
      seq = it - xi * S;
      part = 0;
      const int L = min(len_next, maxlen);
      if (it + 1 < nitems) len_next = a.context_lens[(it + 1) % S];
      const int64_t n = L > 0 ? (L + TT - 1) / TT : 0;
      const int64_t r0 = C + cost;  // the item's first tile
      const int64_t lo = X0 > r0 ? X0 : r0, hi = X1 < r0 + n ? X1 : r0 + n;
      C = r0 + n;
      if (lo >= hi) continue;
      t_lo = (int)(lo - r0);
      t_hi = (int)(hi - r0);
    } else {  // the grid's unit
      xi = blockIdx.x;
      seq = blockIdx.y;
      part = blockIdx.z;
      if (a.unit_order != nullptr) {  // longest-first schedule over a 1-D grid
        const int X = a.num_kv_heads * a.row_chunks;
        int b = blockIdx.x;
        if constexpr (STAGE) {
          // Workgroups of the first round (one per CU) keep their place; each
          // later one takes the next place in the order of its start.  The
          // hardware deals workgroups to the XCDs in turn, so by block index
          // a slower XCD would get as many long units as a faster one; by
          // start order, the CUs that free first take the longer remaining
          // units whatever XCD they sit on (MQA 48/1 ragged batch 256: 103.8
          // -> 98.6 us).  Places are unique and cover the rest of the order,
          // so every unit is still walked exactly once.
          if (a.ticket != nullptr && b >= a.static_wgs) {
            int* tk = reinterpret_cast<int*>(toff_lds);  // (the table window is filled later)
            if (threadIdx.x == 0) *tk = atomicAdd(a.ticket, 1);
            __syncthreads();
            // (a counter the ordering kernel did not clear could only give a
            // wrong place, never one outside the grid)
            const int t = __builtin_amdgcn_readfirstlane(*tk);
            b = a.static_wgs + min(max(t, 0), (int)gridDim.x - 1 - a.static_wgs);
          }
        }
        const int n = b / X;
        const int u = a.unit_order[n];
        xi = b - n * X;
        seq = u % S;
        part = u / S;
      }
      t_lo = part * a.partition_blocks * BS / TT;
      t_hi = t_lo + a.partition_blocks * BS / TT;
    }
    unit(xi, seq, part, t_lo, t_hi, it);
  }
}

namespace {

template <typename Fmt, int D, int NT, int TG, int RT, int KT, bool KV8>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid = a.unit_order != nullptr
                       ? dim3(a.num_kv_heads * a.row_chunks * a.num_seqs * a.num_partitions)
                       : dim3(a.num_kv_heads * a.row_chunks, a.num_seqs, a.num_partitions);
  if constexpr (NT > 1 && RT == 1) {  // decode on the staged kernel
    if (a.stream_wgs > 0) {
      decode_mfma_kernel<Fmt, D, NT, TG, RT, KT, KV8, true><<<a.stream_wgs, NT * TG * 64, 0, s>>>(a);
      return hipGetLastError();
    }
  }
  decode_mfma_kernel<Fmt, D, NT, TG, RT, KT, KV8><<<grid, NT * TG * 64, 0, s>>>(a);
  return hipGetLastError();
}

// Head tiles NT = ceil(G / 16); token groups TG chosen so a workgroup has
// 4 waves where possible; 48-head groups (3 tiles sharing every K/V tile
// through the LDS ring) take 4 token groups, 12 waves (measured against 2:
// MQA ragged batch 256 148 -> 134 us; against 3: 133 -> 126 us).  For one
// head tile, 1-3 token groups were measured slower or, with one group, unfit
// for ragged batches (a whole sequence on one wave).  With an FP8 cache the
// staged decode takes tile pairs (half-size slots; the per-key softmax and
// step overhead, not the bytes, bound it: MQA 124.5 -> 113 us, 64-head groups
// 142 -> 128 us); 16-bit caches keep single tiles (pairs fit only a 2-slot
// ring for 4 token groups: MQA 122 -> 135 us).
template <typename Fmt, int D, bool KV8>
hipError_t launch_g(const DecodeArgs& a, hipStream_t s) {
  // multi-query: kPrefillWaves waves of kPrefillRowTilesPerWave 16-row tiles
  // each, all walking the same keys, in pairs of key tiles
  if (a.query_start != nullptr)
    return launch_t<Fmt, D, kPrefillWaves, 1, kPrefillRowTilesPerWave, 2, KV8>(a, s);
  switch (mfma_head_tiles(a.group)) {
    case 1: return launch_t<Fmt, D, 1, 4, 1, 1, KV8>(a, s);
    case 2: return launch_t<Fmt, D, 2, staged_token_groups(2), 1, KV8 ? 2 : 1, KV8>(a, s);
    case 3: return launch_t<Fmt, D, 3, staged_token_groups(3), 1, KV8 ? 2 : 1, KV8>(a, s);
    default: return launch_t<Fmt, D, 4, staged_token_groups(4), 1, KV8 ? 2 : 1, KV8>(a, s);
  }
}

template <typename Fmt, bool KV8>
hipError_t launch_d(const DecodeArgs& a, int head_size, hipStream_t s) {
  return head_size == 64 ? launch_g<Fmt, 64, KV8>(a, s) : launch_g<Fmt, 128, KV8>(a, s);
}

}  // namespace

namespace {

template <typename Fmt, int D, bool KV8, int NT>
hipError_t occupancy_t(int* wgs) {
  constexpr int TG = staged_token_groups(NT);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(
      wgs, reinterpret_cast<const void*>(decode_mfma_kernel<Fmt, D, NT, TG, 1, KV8 ? 2 : 1, KV8, true>),
      NT * TG * 64, 0);
}
template <typename Fmt, int D, bool KV8>
hipError_t occupancy_g(int group, int* wgs) {
  switch (mfma_head_tiles(group)) {
    case 2: return occupancy_t<Fmt, D, KV8, 2>(wgs);
    case 3: return occupancy_t<Fmt, D, KV8, 3>(wgs);
    default: return occupancy_t<Fmt, D, KV8, 4>(wgs);
  }
}

}  // namespace

hipError_t staged_decode_occupancy(int dtype, int head_size, int group, bool kv_fp8, int* wgs) {
  if (mfma_head_tiles(group) < 2) return hipErrorInvalidValue;
  if (dtype == 0) {
    if (head_size == 64) return kv_fp8 ? occupancy_g<F16, 64, true>(group, wgs) : occupancy_g<F16, 64, false>(group, wgs);
    return kv_fp8 ? occupancy_g<F16, 128, true>(group, wgs) : occupancy_g<F16, 128, false>(group, wgs);
  }
  if (head_size == 64) return kv_fp8 ? occupancy_g<BF16, 64, true>(group, wgs) : occupancy_g<BF16, 64, false>(group, wgs);
  return kv_fp8 ? occupancy_g<BF16, 128, true>(group, wgs) : occupancy_g<BF16, 128, false>(group, wgs);
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int dtype, int head_size, bool kv_fp8,
                              hipStream_t s) {
  if (dtype == 0)
    return kv_fp8 ? launch_d<F16, true>(a, head_size, s) : launch_d<F16, false>(a, head_size, s);
  return kv_fp8 ? launch_d<BF16, true>(a, head_size, s) : launch_d<BF16, false>(a, head_size, s);
}

}  // namespace pa
