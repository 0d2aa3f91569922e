// Paged decode attention on the matrix cores (MFMA) of gfx950: the kernel
// template.  decode_mfma.hip instantiates it and launches it.
//
// Same result as the vector-ALU kernel -- softmax(scale q K^T) V over each
// sequence's paged context with GQA ("[Hacker News 요약] C++와 CUDA로 vLLM의 경량
// 고성능 LLM 추론 엔진 'Tiny-vLLM' 직접 구축하기", section "고성능 추론을 위한 고급
// 최적화 기법"; paging per "vLLM -- PagedAttention으로 LLM 추론 성능을 2~4배
// 끌어올린 서빙 엔진", section "PagedAttention -- OS 가상 메모리에서 영감") -- but the
// two contractions of a 16-token sub-tile run as MFMA tiles, so the vector ALU
// only does the softmax:
//
//   S^T[16 tok x 16 cols] = K[16 tok x D] . Q^T[D x 16 cols]   (D/32 x mfma 16x16x32)
//   O^T[D x 16 cols]     += V^T[D x 16 tok] . P^T[16 tok x 16 cols] (D/16 x mfma 16x16x16)
//
// The 16 columns are the G q heads that share the kv head (G <= 16; unused
// columns hold zero queries).  The pools are token-major ([bs][D] per block
// and kv head), so a 16-token sub-tile is 16 consecutive rows of D values.
// For the K operand lane l = 16*kg + r reads 8 dims (32j + 8kg ..) of token r:
// 16 bytes, a wave instruction covering half of each of the 16 rows.  The V
// operand needs 4 tokens of one dim in a lane, across the rows.  The order of
// the D rows of V^T is free (it only permutes the rows of O^T), so operand j
// of lane l is taken to be dim JV*r + j (JV = D/16): lane l reads dims
// JV*r .. JV*r + JV-1 of tokens 4kg + i, i = 0..3 (one load per i; the 16 lanes
// of a row together read the whole row, so a wave instruction covers 4 full
// rows), and regroups the 16-bit values in its own registers, with no
// cross-lane traffic.  The S tile comes back with lane l holding tokens
// 4kg..4kg+3 of column r, which is exactly the P^T operand layout of the PV
// product, so probabilities never leave registers.
//
// Softmax is online in fp32 (log2 domain).  P enters the PV product rounded to
// the cache's 16-bit type (round to nearest even); the denominator sums the same
// rounded values, so the output is an exact convex combination of V rows up to
// fp32 rounding.  Tokens past the context are masked by select (score -inf, V
// 0), so NaN in tail slots never reaches the output.
//
// Work split: one workgroup per (sequence, kv head, partition); its NW waves
// take the partition's 16-token sub-tiles round robin (wave w: w, w+NW, ...).
// Decode moves every cached byte once and does little arithmetic on it, so the
// kernel is organised around keeping HBM busy: each wave keeps S sub-tiles
// (S * 4 KB at D = 64) in flight, refilling a register slot as soon as its
// sub-tile has been consumed, and every wave fetches the physical ids of all
// its sub-tiles with one load at the start (one id per lane, read back with
// readlane), so the only dependent HBM round trip is the block-table read.
//
// Partitions of one (sequence, kv head) store their softmax states and the
// merge kernel (merge.hip) folds them.
//
// Optionally the kernel also performs the step's KV append (see the fused
// append block below), so a decode step is one launch per layer.
#pragma once

#include <type_traits>

#include "decode_common.h"

namespace pkv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename T> struct Mma;

template <> struct Mma<Bf16> {
  typedef __bf16 x8 __attribute__((ext_vector_type(8)));
  typedef short x4 __attribute__((ext_vector_type(4)));
  typedef __bf16 x2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(x8, a), __builtin_bit_cast(x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(x4, a), __builtin_bit_cast(x4, b), c, 0, 0,
                                                     0);
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, x2));
  }
  // a + lo(w) + hi(w) for a word of two bf16 values (one dot2 instruction)
  static __device__ __forceinline__ float sum2(uint32_t w, float a) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(x2, w), __builtin_bit_cast(x2, 0x3f803f80u), a, false);
  }
};

template <> struct Mma<Fp16> {
  typedef _Float16 x8 __attribute__((ext_vector_type(8)));
  typedef _Float16 x4 __attribute__((ext_vector_type(4)));
  typedef _Float16 x2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(x8, a), __builtin_bit_cast(x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(x4, a), __builtin_bit_cast(x4, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, x2));
  }
  static __device__ __forceinline__ float sum2(uint32_t w, float a) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(x2, w), __builtin_bit_cast(x2, 0x3c003c00u), a, false);
  }
};

// Word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data, no
// swizzle); with stride 0 and range 0xffffffff the buffer is a plain byte range.
constexpr int kBufferConfig = 0x00020000;

// D/16 16-bit values of one token: the slice of a V row one lane reads.
template <int D> struct VSlice;
template <> struct VSlice<64> {
  u32x2 w;
  static __device__ __forceinline__ VSlice load(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
    return VSlice{__builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0))};
  }
};
template <> struct VSlice<128> {
  u32x4 w;
  static __device__ __forceinline__ VSlice load(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
    return VSlice{__builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0))};
  }
};

// The registers one sub-tile needs: K operands (one per 32 dims) and, for V,
// the row slices of the lane's 4 tokens.
template <int D> struct Tile {
  u32x4 k[D / 32];
  VSlice<D> v[4];
};

// PV operand j from the 4 row slices: dim JV*r + j of tokens 0..3 as
// {t0 t1 | t2 t3} (16 bits each, low half first).
template <int D>
__device__ __forceinline__ u32x2 v_operand(const VSlice<D> (&v)[4], int j) {
  const int w = j >> 1;
  // byte permute: the low (j even) or high (j odd) 16-bit halves of two words
  const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
  return u32x2{__builtin_amdgcn_perm(v[1].w[w], v[0].w[w], sel), __builtin_amdgcn_perm(v[3].w[w], v[2].w[w], sel)};
}

// Fused append, store side (the pools are writable for fused calls; the
// parameter block keeps them const to stay small): the same bytes kv_append writes for token i =
// sequence i, after the checks the decode side makes (a valid length, and the
// slot is the slot of position L_i - 1); thread per (token, kv head, 8-dim run)
// as in kv_append, grid-strided over the append workgroups.  A token's K and V
// are one D-value row each.
template <int D, int NT>
__device__ __forceinline__ void append_tokens(const DecodeParams& p) {
  constexpr int runs = D / 8;
  const int64_t total = static_cast<int64_t>(p.num_seqs) * p.num_kv_heads * runs;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x; i < total;
       i += static_cast<int64_t>(p.append_wgs) * NT) {
    const int c = static_cast<int>(i % runs);
    const int64_t th = i / runs;  // sequence * Hkv + kv head
    const int h = static_cast<int>(th % p.num_kv_heads);
    const int t = static_cast<int>(th / p.num_kv_heads);
    const int64_t slot = p.slot_mapping[t];
    const int L = p.context_lens[t];
    if (slot < 0 || L <= 0 || bad_length(L, p)) continue;
    const int pos = L - 1;
    const int blk = pos / p.block_size;
    const int phys = p.block_tables[static_cast<size_t>(t) * p.max_blocks_per_seq + blk];
    const int off = pos - blk * p.block_size;
    if (static_cast<unsigned>(phys) >= static_cast<unsigned>(p.num_blocks) ||
        slot != static_cast<int64_t>(phys) * p.block_size + off)
      continue;
    const size_t row = ((static_cast<size_t>(phys) * p.num_kv_heads + h) * p.block_size + off) * D + c * 8;
    *reinterpret_cast<u32x4*>(const_cast<uint16_t*>(p.k_cache) + row) = *reinterpret_cast<const u32x4*>(p.k_new + th * D + c * 8);
    *reinterpret_cast<u32x4*>(const_cast<uint16_t*>(p.v_cache) + row) = *reinterpret_cast<const u32x4*>(p.v_new + th * D + c * 8);
  }
}

// Shared prefixes read once per prefix item.  Sequences whose block tables
// start with the same physical blocks hold the same K/V there (blocks are
// shared by reference, "Nano-vLLM로 배우는 vLLM 추론 엔진 작동 원리 한눈에 정리",
// section "KV 캐시와 Block Manager").  A prefix item puts up to CG * 16/G of
// them into the MFMA columns -- column (cg, r) is member cg*16/G + r/G, q
// head kvh*G + r%G -- and one wave streams a chunk of the reference member's
// shared blocks for all of them, each column masked at its own member's
// prefix length.  It writes each member's softmax state over the chunk into
// the partial-state slot num_parts + chunk; the merge folds those with the
// states of the member's regular partitions, which start after the prefix.
//
// Before the first sub-tile the wave checks, block by block, that every
// member's table names the reference's block wherever it reads that member's
// prefix; a member that differs (or claims more prefix than the reference,
// or whose reference is unusable) gets NaN in its state, so a wrong plan
// shows as NaN output rather than as another sequence's attention.
//
// Masked keys contribute probability 0 but are multiplied into P.V, so a
// non-finite V value in a reference block past a member's prefix length would
// reach that member; cached values are finite.
template <typename T, int D, int G>
__device__ __forceinline__ void prefix_unit(const DecodeParams& p, const DecodeExt& x, int unit) {
  constexpr int JK = D / 32, JV = D / 16;
  constexpr int CG = prefix_column_groups(D, G);
  constexpr int MPC = 16 / G;     // members per column group
  constexpr int NM = CG * MPC;    // members per item, <= 16
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15, kg = lane >> 4;
  const int chunk = unit % x.prefix_chunks;
  unit /= x.prefix_chunks;
  const int kvh = unit % p.num_kv_heads;
  const int item = unit / p.num_kv_heads;
  if (item >= x.num_prefix_items) return;
  const int32_t* mem = x.prefix_items + static_cast<size_t>(item) * 16;
  const int c0 = chunk * x.prefix_chunk;

  // the reference member and its usable prefix length (-1: unusable)
  const int ref = mem[0];
  int ref_lim = -1;
  if (static_cast<unsigned>(ref) < static_cast<unsigned>(p.num_seqs)) {
    const int Lr = p.context_lens[ref];
    if (!bad_length(Lr, p)) ref_lim = seq_prefix(x, ref, Lr);
  }

  // lane mi < NM: member mi's sequence and prefix length; mlim = 0: no prefix
  // part here (absent, no prefix, or an unusable length, which the regular
  // items turn into NaN themselves); mbad: a prefix this item cannot serve
  int ms = -1, mlim = 0;
  bool mbad = false;
  if (lane < NM) {
    const int sq = mem[lane];
    if (static_cast<unsigned>(sq) < static_cast<unsigned>(p.num_seqs)) {
      const int L = p.context_lens[sq];
      const int pl = bad_length(L, p) ? 0 : seq_prefix(x, sq, L);
      if (pl > 0) {
        ms = sq;
        mlim = pl;
        mbad = pl > ref_lim;
      }
    }
  }
  if (ref_lim <= c0) {
    // nothing of the reference in this chunk: only chunk 0 reports the
    // members this item cannot serve
    if (chunk != 0) return;
  }
  const int c1 = ref_lim > c0 ? min(c0 + x.prefix_chunk, ref_lim) : c0;
  const int nsub = (c1 - c0) >> 4;

  // block-by-block check of the members' tables against the reference row
  // over this chunk (at most 64 blocks: the chunk is at most 1024 tokens)
  const int b0 = c0 / p.block_size;
  const int nb = nsub > 0 ? (c1 - 1) / p.block_size - b0 + 1 : 0;
  const size_t mrow = static_cast<size_t>(p.max_blocks_per_seq);
  int refb = -1;
  if (lane < nb) refb = p.block_tables[static_cast<size_t>(ref) * mrow + b0 + lane];
  int ent[NM];
#pragma unroll
  for (int mi = 1; mi < NM; ++mi) {
    const int sq = __builtin_amdgcn_readlane(ms, mi);
    const int lm = __builtin_amdgcn_readlane(mlim, mi);
    const int nbm = lm > c0 && nsub > 0 ? (min(c1, lm) - 1) / p.block_size - b0 + 1 : 0;
    ent[mi] = refb;
    if (lane < nbm) ent[mi] = p.block_tables[static_cast<size_t>(sq) * mrow + b0 + lane];
  }
#pragma unroll
  for (int mi = 1; mi < NM; ++mi)
    if (__builtin_amdgcn_ballot_w64(ent[mi] != refb)) mbad = mbad || lane == mi;

  // the columns: member cg*MPC + r/G of this lane's column group cg
  int lim[CG], seqc[CG];
  bool cbad[CG];
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) {
    const int mi = cg * MPC + r / G;
    seqc[cg] = __shfl(ms, mi, kWave);
    lim[cg] = __shfl(mlim, mi, kWave);
    cbad[cg] = __shfl(static_cast<int>(mbad), mi, kWave) != 0;
  }
  const int head = kvh * G + r % G;
  u32x4 qop[CG][JK];
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) {
#pragma unroll
    for (int j = 0; j < JK; ++j) {
      if (lim[cg] > c0 && !cbad[cg]) {
        qop[cg][j] = *reinterpret_cast<const u32x4*>(
            p.q + (static_cast<size_t>(seqc[cg]) * p.num_q_heads + head) * D + (kg + 4 * j) * 8);
      } else {
        qop[cg][j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  // pool index of the chunk's sub-tiles, one per lane (-1: outside the pool)
  int tid = 0;
  if (lane < nsub) {
    const int tok0 = c0 + 16 * lane;
    const int blk = tok0 / p.block_size;
    const int phys = p.block_tables[static_cast<size_t>(ref) * mrow + blk];
    tid = static_cast<unsigned>(phys) < static_cast<unsigned>(p.num_blocks)
              ? (phys * p.num_kv_heads + kvh) * (p.block_size >> 4) + ((tok0 - blk * p.block_size) >> 4)
              : -1;
  }
  bool bad = false;
  const int koff = (r * D + kg * 8) * 2;
  const int voff = (4 * kg * D + r * JV) * 2;
  auto load = [&](int k, Tile<D>& t) {
    int sub = __builtin_amdgcn_readlane(tid, k);
    bad |= sub < 0;
    sub = max(sub, 0);
    const uint16_t* kt = p.k_cache + static_cast<size_t>(sub) * (16 * D);
    const uint16_t* vt = p.v_cache + static_cast<size_t>(sub) * (16 * D);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kt), 0, -1, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vt), 0, -1, kBufferConfig);
#pragma unroll
    for (int j = 0; j < JK; ++j)
      t.k[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, koff, 64 * j, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) t.v[i] = VSlice<D>::load(rv, voff, i * D * 2);
  };

  float m[CG], l[CG];
  f32x4 o[CG][JV];
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) {
    m[cg] = -INFINITY;
    l[cg] = 0.f;
#pragma unroll
    for (int j = 0; j < JV; ++j) o[cg][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // every key of the chunk is a prefix token of the reference; key t counts
  // for column (cg, r) when t < lim[cg].  A column with no key yet keeps
  // m = -inf, and its exponents are taken against 0 instead.
  auto compute = [&](int k, Tile<D>& t) {
    const int key0 = c0 + 16 * k;
    u32x2 vop[JV];
#pragma unroll
    for (int j = 0; j < JV; ++j) vop[j] = v_operand<D>(t.v, j);
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < JK; ++j) sc = Mma<T>::qk(t.k[j], qop[cg][j], sc);
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = key0 + 4 * kg + i < lim[cg] ? sc[i] * p.scale_log2 : -INFINITY;
      float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      bm = max_xor32(max_xor16(bm));
      const float mn = fmaxf(m[cg], bm);
      const float mref = mn == -INFINITY ? 0.f : mn;
      const float al = fast_exp2(m[cg] - mref);
      m[cg] = mn;
      const uint32_t p01 = Mma<T>::pack(fast_exp2(x[0] - mref), fast_exp2(x[1] - mref));
      const uint32_t p23 = Mma<T>::pack(fast_exp2(x[2] - mref), fast_exp2(x[3] - mref));
      l[cg] = Mma<T>::sum2(p23, Mma<T>::sum2(p01, l[cg] * al));
      if (__builtin_amdgcn_ballot_w64(al != 1.f)) {
#pragma unroll
        for (int j = 0; j < JV; ++j) o[cg][j] *= al;
      }
      const u32x2 pop = {p01, p23};
#pragma unroll
      for (int j = 0; j < JV; ++j) o[cg][j] = Mma<T>::pv(vop[j], pop, o[cg][j]);
    }
  };

  if (nsub > 0) {
    Tile<D> t[2];
    const int last = nsub - 1;
    load(0, t[0]);
    load(min(1, last), t[1]);
    const int n_pad = (nsub + 1) & ~1;
    int kb = 0;
    for (; kb + 2 < n_pad; kb += 2) {
      compute(kb, t[0]);
      load(min(kb + 2, last), t[0]);
      compute(kb + 1, t[1]);
      load(min(kb + 3, last), t[1]);
    }
    compute(kb, t[0]);
    if (kb + 1 < nsub) compute(kb + 1, t[1]);
  }

  // lane (kg, r) holds rows 4kg+i of O^T for column r: dims (4kg+i)*JV + j
  const size_t slot = static_cast<size_t>(p.num_parts) + chunk;
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) {
    float lt = add_xor32(add_xor16(l[cg]));
    const bool has_keys = lim[cg] > c0 && nsub > 0;
    // a member this item cannot serve is reported in its chunk-0 state
    const bool report = cbad[cg] && chunk == 0;
    if (!has_keys && !report) continue;
    if (bad || cbad[cg]) lt = __int_as_float(0x7fc00000);
    const size_t pr = (static_cast<size_t>(seqc[cg]) * p.num_q_heads + head) * x.num_slots + slot;
    if (kg == 0) {
      p.part_m[pr] = m[cg];
      p.part_l[pr] = lt;
    }
#pragma unroll
    for (int j = 0; j < JV; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) p.part_o[pr * D + (4 * kg + i) * JV + j] = o[cg][j][i];
  }
}

// Waves with more sub-tiles than this run the deep register ring (S slots),
// the others a two-slot ring.
constexpr int kDeepRingSubTiles = 16;

// MINW: waves per SIMD the register allocation must allow; the launcher picks
// S and MINW per head size so that nothing spills.  At most three waves per
// SIMD: with the head_dim 64 tile the allocation would otherwise fit four,
// which measured slower on the Llama-3.2-1B batch.
// EXT: the launch may have shared-prefix units (x.prefix_len), a work list
// (x.work) and wave-mode entries; the kernel without them carries none of
// their code (the plain decode keeps its registers and instruction stream).
template <typename T, int D, int G, int NW, int S, bool EXT>
__device__ __forceinline__ void decode_body(const DecodeParams& p, const DecodeExt& x) {
  constexpr int JK = D / 32, JV = D / 16;
  __shared__ float sm_m[NW][G], sm_l[NW][G], sm_o[NW][G][D];

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int r = lane & 15, kg = lane >> 4;
  if (static_cast<int>(blockIdx.x) < p.append_wgs) {
    append_tokens<D, NW * kWave>(p);
    return;
  }
  const int pb = static_cast<int>(blockIdx.x) - p.append_wgs;
  constexpr bool PREFIX = EXT;
  const int prefix_wgs = PREFIX ? x.prefix_wgs : 0;
  if (PREFIX && pb < prefix_wgs) {
    // shared-prefix units, one per wave (no workgroup barrier on this path)
    prefix_unit<T, D, G>(p, x, xcd_remap(pb, prefix_wgs) * NW + wv);
    return;
  }
  const int nreg = static_cast<int>(gridDim.x) - p.append_wgs - prefix_wgs;
  WorkItem w = decode_item<EXT>(p, pb - prefix_wgs, nreg, x);
  if (w.seq < 0) return;
  // Wave mode (a short partition from a work list): wave wv takes kv head
  // kvh + wv alone, all the partition's sub-tiles, and stores its own state;
  // no wave of such a workgroup reaches a workgroup barrier.
  const bool wmode = EXT && w.wave;
  if (wmode) {
    w.kvh += wv;
    if (w.kvh >= p.num_kv_heads) return;
  }
  const int L = p.context_lens[w.seq];
  const bool bad_len = bad_length(L, p);
  // positions before pl are the sequence's shared prefix, read by the prefix units
  const int pl = !PREFIX || bad_len ? 0 : seq_prefix(x, w.seq, L);
  if (bad_len || L == 0 || pl < 0) {
    // an appended token needs a position: L = 0 with a slot is a caller error
    const bool orphan = p.slot_mapping != nullptr && p.slot_mapping[w.seq] >= 0;
    if (wmode) {
      write_degenerate<T, G, NW * kWave>(p, w, bad_len || orphan || pl < 0, lane, kWave);
    } else {
      write_degenerate<T, G, NW * kWave>(p, w, bad_len || orphan || pl < 0);
    }
    return;
  }
  const int start = pl + w.part * p.part_tokens;
  if (start >= L) return;
  const int end = min(L, start + p.part_tokens);
  const int nsub = (end - start + 15) >> 4;
  const int nparts = (L - pl + p.part_tokens - 1) / p.part_tokens;
  // this wave owns sub-tiles sb + k*ss, k = 0 .. n_w-1: wv + k*NW, or in wave
  // mode all of them (at most the 64 a wave holds ids for: more is an error)
  const int sb = wmode ? 0 : wv, ss = wmode ? 1 : NW;
  const bool too_long = wmode && nsub > kWave;
  const int n_w = wmode ? min(nsub, kWave) : (wv < nsub ? (nsub - wv + NW - 1) / NW : 0);

  // Q^T operand: column r = q head kvh*G + r (zero for r >= G), dims of run kg + 4j
  u32x4 qop[JK];
#pragma unroll
  for (int j = 0; j < JK; ++j) {
    if (r < G) {
      qop[j] = *reinterpret_cast<const u32x4*>(
          p.q + (static_cast<size_t>(w.seq) * p.num_q_heads + w.kvh * G + r) * D + (kg + 4 * j) * 8);
    } else {
      qop[j] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // K and V of the token appended this step (fused append, below); read
  // before the block-table window so that both are in flight together.
  // The slot and the physical block of position L-1 are read here too, so the
  // check below costs no round trip of its own.
  // Lane c < D/8 holds K dims 8c .. 8c+7, lane c < 16 the V dims of row slice c.
  u32x4 krun = {0u, 0u, 0u, 0u};
  VSlice<D> vrun{};
  int64_t app_slot = -1;
  int app_phys = 0;
  if (p.slot_mapping != nullptr) {
    const size_t row = static_cast<size_t>(w.seq) * p.num_kv_heads + w.kvh;
    krun = *reinterpret_cast<const u32x4*>(p.k_new + row * D + 8 * min(lane, D / 8 - 1));
    vrun = *reinterpret_cast<const VSlice<D>*>(p.v_new + row * D + JV * r);
    app_slot = p.slot_mapping[w.seq];
    app_phys = p.block_tables[static_cast<size_t>(w.seq) * p.max_blocks_per_seq + (L - 1) / p.block_size];
  }

  // lane k: index of this wave's k-th sub-tile in the pool (sub-tiles of 16*D
  // elements, numbered (block*Hkv + kvh)*(bs/16) + sub-tile in block), or -1
  // when the table names a block outside the pool.
  int tid = 0;
  if (lane < n_w) {
    const int tok0 = start + 16 * (sb + lane * ss);
    const int blk = tok0 / p.block_size;
    const int phys = p.block_tables[static_cast<size_t>(w.seq) * p.max_blocks_per_seq + blk];
    tid = static_cast<unsigned>(phys) < static_cast<unsigned>(p.num_blocks)
              ? (phys * p.num_kv_heads + w.kvh) * (p.block_size >> 4) + ((tok0 - blk * p.block_size) >> 4)
              : -1;
  }
  bool bad = too_long;

  // Fused append of the token decoded this step, which sits at position L-1.
  // Its K and V were read together with the block-table window, so the
  // append adds no dependent round trip before the first sub-tile loads.  In
  // the workgroup whose partition holds L-1, the wave that reads that sub-tile
  // stages the token in LDS of its own (no workgroup barrier) and puts it into
  // its registers in place of whatever the load returned; the launch's leading
  // append workgroups store it into the pools (append_tokens).  The slot is
  // checked against the block the table names for L-1 after the sub-tile loop,
  // so nothing before the first loads waits for that block id; a slot that is
  // not the slot of L-1 is not written and makes the sequence's output NaN
  // (every workgroup of the sequence checks).
  // the appended token's K and V; one copy per wave in wave mode, where the
  // waves hold different kv heads
  __shared__ __align__(16) uint16_t sm_new[EXT ? NW : 1][2][D];
  const int sw = EXT ? wv : 0;            // this wave's copy
  int app_w = -1, app_k = -1, app_r = 0;  // wave, step and token row that hold it
  if (p.slot_mapping != nullptr && app_slot >= 0) {
    const int app_pos = L - 1;
    if (app_pos >= start && app_pos < end) {
      app_r = app_pos & 15;  // the block size is a multiple of 16
      const int s_tok = (app_pos - start) >> 4;
      app_w = wmode ? wv : s_tok % NW;
      app_k = wmode ? s_tok : s_tok / NW;
      if (wv == app_w) {
        if (lane < D / 8) *reinterpret_cast<u32x4*>(&sm_new[sw][0][8 * lane]) = krun;
        if (lane < 16) *reinterpret_cast<VSlice<D>*>(&sm_new[sw][1][JV * lane]) = vrun;
        // the same wave reads the rows back in its compute step
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
  }

  // Branch-free, so that every path issues the same loads and the compiler's
  // wait counts keep S-1 sub-tiles in flight.  A bad block id makes the
  // whole head group NaN, so what is read in its place (sub-tile 0 of the
  // pool, always in bounds) does not matter.
  //
  // Buffer loads: the sub-tile's base address lives in a wave-uniform
  // resource (scalar registers) and each lane keeps two constant byte
  // offsets, so no per-load address occupies vector registers.
  const int koff = (r * D + kg * 8) * 2;        // K token r, dims 8kg..; + 64 B (scalar offset) per j
  const int voff = (4 * kg * D + r * JV) * 2;   // V token 4kg, dims JV*r..; + one row (scalar offset) per token
  auto load = [&](int k, Tile<D>& t) {
    int sub = __builtin_amdgcn_readlane(tid, k);
    bad |= sub < 0;
    sub = max(sub, 0);
    const uint16_t* kt = p.k_cache + static_cast<size_t>(sub) * (16 * D);
    const uint16_t* vt = p.v_cache + static_cast<size_t>(sub) * (16 * D);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kt), 0, -1, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vt), 0, -1, kBufferConfig);
#pragma unroll
    for (int j = 0; j < JK; ++j)
      t.k[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, koff, 64 * j, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) t.v[i] = VSlice<D>::load(rv, voff, i * D * 2);
  };

  float m = -INFINITY, l = 0.f;
  f32x4 o[JV];
#pragma unroll
  for (int j = 0; j < JV; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // k-th sub-tile of this wave; k >= n_w is an empty pad step (every token
  // masked), which leaves the state unchanged since k = 0 is never empty.
  auto compute = [&](int k, Tile<D>& t) {
    if (k == app_k && wv == app_w) {
      // token row app_r of this sub-tile is the appended token
      if (r == app_r) {
#pragma unroll
        for (int j = 0; j < JK; ++j) t.k[j] = *reinterpret_cast<const u32x4*>(&sm_new[sw][0][(4 * j + kg) * 8]);
      }
      if ((app_r >> 2) == kg) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((app_r & 3) == i) t.v[i] = *reinterpret_cast<const VSlice<D>*>(&sm_new[sw][1][r * JV]);
      }
    }
    u32x2 vop[JV];
#pragma unroll
    for (int j = 0; j < JV; ++j) vop[j] = v_operand<D>(t.v, j);
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < JK; ++j) sc = Mma<T>::qk(t.k[j], qop[j], sc);
    const int nvalid = k < n_w ? min(16, end - (start + 16 * (sb + k * ss))) : 0;
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = 4 * kg + i < nvalid ? sc[i] * p.scale_log2 : -INFINITY;
    float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    bm = max_xor32(max_xor16(bm));
    const float mn = fmaxf(m, bm);
    const float al = fast_exp2(m - mn);
    m = mn;
    const uint32_t p01 = Mma<T>::pack(fast_exp2(x[0] - mn), fast_exp2(x[1] - mn));
    const uint32_t p23 = Mma<T>::pack(fast_exp2(x[2] - mn), fast_exp2(x[3] - mn));
    l = Mma<T>::sum2(p23, Mma<T>::sum2(p01, l * al));
    if (__builtin_amdgcn_ballot_w64(al != 1.f)) {
#pragma unroll
      for (int j = 0; j < JV; ++j) o[j] *= al;
    }
    if (nvalid < 16) {
      const uint32_t m0 = (4 * kg < nvalid ? 0xffffu : 0u) | (4 * kg + 1 < nvalid ? 0xffff0000u : 0u);
      const uint32_t m1 = (4 * kg + 2 < nvalid ? 0xffffu : 0u) | (4 * kg + 3 < nvalid ? 0xffff0000u : 0u);
#pragma unroll
      for (int j = 0; j < JV; ++j) {
        vop[j].x &= m0;
        vop[j].y &= m1;
      }
    }
    const u32x2 pop = {p01, p23};
#pragma unroll
    for (int j = 0; j < JV; ++j) o[j] = Mma<T>::pv(vop[j], pop, o[j]);
  };

  // SS register slots; slot i holds sub-tiles i, i+SS, i+2SS, ...  Steps past
  // n_w re-load the wave's last sub-tile (a cache hit) and compute it as an
  // empty pad step, so the loop body is the same straight-line code every
  // time and the compiler's wait counts stay SS-1 sub-tiles deep.
  auto ring = [&](auto depth) {
    constexpr int SS = decltype(depth)::value;
    Tile<D> t[SS];
    const int last = n_w - 1;
#pragma unroll
    for (int i = 0; i < SS; ++i) load(min(i, last), t[i]);
    const int n_pad = (n_w + SS - 1) / SS * SS;
    int kb = 0;
    for (; kb + SS < n_pad; kb += SS) {
#pragma unroll
      for (int i = 0; i < SS; ++i) {
        compute(kb + i, t[i]);
        load(min(kb + i + SS, last), t[i]);
      }
    }
    // the final round: pad steps leave the state unchanged, so they are
    // skipped (a wave-uniform branch after the last loads, where the wait
    // counts no longer matter)
#pragma unroll
    for (int i = 0; i < SS; ++i)
      if (kb + i < n_w) compute(kb + i, t[i]);
  };
  // A deep ring pays only when a wave has many sub-tiles: with few, its pad
  // steps (up to SS-1 per wave) cost more than the extra loads in flight gain,
  // and the other waves of the compute unit keep HBM busy.  Measured on the
  // Llama-3.2-1B batch (at most 16 sub-tiles per wave): two slots 1.1 us faster
  // than four; with 32 sub-tiles per wave (the long-context partitions) four
  // slots are 0.8 us faster.
  if (n_w > kDeepRingSubTiles) {
    ring(std::integral_constant<int, S>{});
  } else if (n_w > 0) {
    ring(std::integral_constant<int, (S < 2 ? S : 2)>{});
  }

  if (p.slot_mapping != nullptr && app_slot >= 0) {
    const int app_pos = L - 1;
    const int off = app_pos - (app_pos / p.block_size) * p.block_size;
    if (static_cast<unsigned>(app_phys) >= static_cast<unsigned>(p.num_blocks) ||
        app_slot != static_cast<int64_t>(app_phys) * p.block_size + off)
      bad = true;
  }

  // fold the four token rows (kg) of the denominator
  l = add_xor32(add_xor16(l));
  if (bad) l = __int_as_float(0x7fc00000);
  if (wmode) {
    // the wave's state is the partition's: lane (kg, r) holds rows 4kg+i of
    // O^T for column r, i.e. dims (4kg+i)*JV + j of q head kvh*G + r
    if (r < G) {
      const size_t row = static_cast<size_t>(w.seq) * p.num_q_heads + w.kvh * G + r;
      if (nparts == 1 && pl == 0) {
        const float inv = 1.f / l;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t wd[JV / 2];
#pragma unroll
          for (int j = 0; j < JV / 2; ++j)
            wd[j] = static_cast<uint32_t>(to_bits<T>(o[2 * j][i] * inv)) |
                    (static_cast<uint32_t>(to_bits<T>(o[2 * j + 1][i] * inv)) << 16);
          uint16_t* dst = p.out + row * D + (4 * kg + i) * JV;
          if constexpr (JV == 4) {
            *reinterpret_cast<u32x2*>(dst) = u32x2{wd[0], wd[1]};
          } else {
            *reinterpret_cast<u32x4*>(dst) = u32x4{wd[0], wd[1], wd[2], wd[3]};
          }
        }
      } else {
        const size_t pr = row * x.num_slots + w.part;
        if (kg == 0) {
          p.part_m[pr] = m;
          p.part_l[pr] = l;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < JV; ++j) p.part_o[pr * D + (4 * kg + i) * JV + j] = o[j][i];
      }
    }
    return;
  }
  if (r < G) {
    if (kg == 0) {
      sm_m[wv][r] = m;
      sm_l[wv][r] = l;
    }
#pragma unroll
    for (int j = 0; j < JV; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_o[wv][r][(4 * kg + i) * JV + j] = o[j][i];  // row 4kg+i of O^T is that dim
  }
  __syncthreads();
  combine_and_store<T, D, G, NW>(sm_m, sm_l, sm_o, p, w, nparts == 1 && pl == 0, EXT ? x.num_slots : p.num_parts);
}

template <typename T, int D, int G, int NW, int S, int MINW>
__global__ __attribute__((amdgpu_flat_work_group_size(1, NW * kWave), amdgpu_waves_per_eu(MINW, 3))) void
decode_mfma_kernel(DecodeParams p) {
  decode_body<T, D, G, NW, S, false>(p, DecodeExt{});
}

// The same with the launch's extensions (shared prefixes, a work list).
template <typename T, int D, int G, int NW, int S, int MINW>
__global__ __attribute__((amdgpu_flat_work_group_size(1, NW * kWave), amdgpu_waves_per_eu(MINW, 3))) void
decode_mfma_ext_kernel(DecodeParams p, DecodeExt x) {
  decode_body<T, D, G, NW, S, true>(p, x);
}

}  // namespace pkv
