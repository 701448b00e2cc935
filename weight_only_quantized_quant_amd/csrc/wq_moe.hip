// W4A8 mixture-of-experts path for gfx950: routing, grouping of the
// (token, expert) pairs by expert, the fp8 recipe for the INT4 group scales,
// and the grouped GEMM whose INT4 weights become E4M3 through a per-group
// byte table and meet E4M3 activations on fp8 MFMA.
//
// Routing: one wave per token with lane e holding expert e's logit; softmax by
// butterfly reductions (every lane ends with the same sum); top-k by k rounds
// of a wave argmax in which equal logits resolve towards the lower expert id.
// Grouping: one workgroup per expert counts the pairs that chose a lower
// expert (its first row) and walks the tokens in order, placing the tokens
// that chose it with a block-wide prefix sum: rows of an expert are in
// increasing token order, and no atomics are involved.
//
// Tables: for an fp8 group scale v there are 16 products w * v over the INT4
// codes w.  A lane keeps them as two 8-byte pools (codes for w = 0..7, and for
// w = -8..-1, the latter being the positive magnitudes with the sign bit
// flipped, exact since rounding to nearest even is sign-symmetric) and looks a
// nibble up with v_perm_b32 in each pool and one more v_perm_b32 keyed on the
// nibble's sign bit.  The weights are re-laid once so that the even nibble
// slots of a word hold its elements 0..3 and the odd slots 4..7: one shift and
// one mask then give four table indices in k order.
//
// Grouped GEMM: 256 x 256 tiles of (rows of one expert) x (output channels),
// 8 waves of 256 x 32, K step 128 = one INT4 group, three LDS stages filled by
// direct-to-LDS loads two steps ahead; the activation rows are gathered through
// row_token.
// v_mfma_scale_f32_32x32x64_f8f6f4 with neutral block scales multiplies the
// E4M3 operands; the epilogue applies the per-token and per-channel fp32
// scales and rounds to bf16 once.  The fp8 MFMA treats E4M3 subnormal
// operands as zero.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "wq.h"
#include "wq_device.h"
#include "wq_host.h"

using namespace wq;

namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Routing and grouping
// ---------------------------------------------------------------------------
// One wave per token, lane e holding logit e (E <= 64).  The softmax maximum
// and sum are xor butterflies over the wave.  The top k follow from each
// expert's rank: the number of experts with a larger logit plus those with an
// equal logit and a lower id (the order of the oracle's stable sort), counted
// by every lane against the token's logits staged in the wave's own LDS row
// (read as broadcasts).  The lanes ranked below k write themselves to
// position rank.  Lanes past E hold -inf, which no finite logit ranks below.
__global__ __launch_bounds__(256) void k_route(const float* __restrict__ logits, int64_t T, int E, int k,
                                               int32_t* __restrict__ ids, float* __restrict__ wts) {
  __shared__ __attribute__((aligned(16))) float zs[4][64];
  const int lane = threadIdx.x & 63, wl = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wl;
  if (t >= T) return;                                   // whole wave; no workgroup barrier below
  const bool valid = lane < E;
  const float z = valid ? logits[t * E + lane] : -INFINITY;
  zs[wl][lane] = z;
  float m = z;
  for (int o = 1; o < 64; o <<= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o, 64));
  const float p = valid ? expf(z - m) : 0.0f;
  float sum = p;
  for (int o = 1; o < 64; o <<= 1) sum += __shfl_xor(sum, o, 64);
  // the wave's LDS accesses execute in order: the row is complete here
  int rank = 0;
#pragma unroll
  for (int j = 0; j < 64; j += 4) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(&zs[wl][j]);
#pragma unroll
    for (int i = 0; i < 4; i++) rank += (v[i] > z || (v[i] == z && j + i < lane)) ? 1 : 0;
  }
  if (valid && rank < k) {
    ids[t * k + rank] = lane;
    wts[t * k + rank] = p / sum;
  }
}

// One workgroup per expert e; wave w owns the w-th of 16 contiguous ranges of
// the T*k (token, slot) pairs, read 64 consecutive pairs per load, a block of
// GROUP_ROUNDS loads in flight at once.  Pass 1 counts, per wave, the pairs
// with an expert below e (the workgroup's sum is the expert's first grouped
// row) and those with expert e; pass 2 places each match at the running
// position of the wave (ballot and popcount), so the rows of e come out in
// increasing pair order, which is increasing token order.  When a wave's
// range is one block (up to 32768 pairs, 4096 tokens x 8) it stays in
// registers for pass 2.
constexpr int GROUP_ROUNDS = 32;
__device__ __forceinline__ void group_load(const int32_t* __restrict__ ids, int64_t base, int64_t p1, int lane,
                                           int (&v)[GROUP_ROUNDS]) {
#pragma unroll
  for (int u = 0; u < GROUP_ROUNDS; u++) {
    const int64_t i = base + 64 * u + lane;
    v[u] = i < p1 ? ids[i] : 0x7FFFFFFF;                // past the range: neither below e nor e
  }
}
__device__ __forceinline__ void group_count(const int (&v)[GROUP_ROUNDS], int e, int& lt, int& cnt) {
#pragma unroll
  for (int u = 0; u < GROUP_ROUNDS; u++) {
    lt += v[u] < e ? 1 : 0;
    cnt += v[u] == e ? 1 : 0;
  }
}
__device__ __forceinline__ void group_place(const int (&v)[GROUP_ROUNDS], int e, int k, int64_t base, int lane,
                                            int& pos, int32_t* __restrict__ row_token,
                                            int32_t* __restrict__ row_slot) {
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int u = 0; u < GROUP_ROUNDS; u++) {
    const bool hit = v[u] == e;
    const unsigned long long b = __ballot(hit);
    if (hit) {
      const int64_t i = base + 64 * u + lane;
      const int r = pos + __popcll(b & below);
      row_token[r] = (int32_t)(i / k);
      row_slot[r] = (int32_t)(i % k);
    }
    pos += __popcll(b);
  }
}
__global__ __launch_bounds__(1024) void k_group(const int32_t* __restrict__ ids, int64_t T, int E, int k,
                                                int32_t* __restrict__ offsets, int32_t* __restrict__ row_token,
                                                int32_t* __restrict__ row_slot) {
  __shared__ int lt_w[16], m_w[16];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t P = T * k;
  const int64_t per = ((P + 15) / 16 + 63) / 64 * 64;
  const int64_t p0 = wv * per < P ? wv * per : P;
  const int64_t p1 = p0 + per < P ? p0 + per : P;
  constexpr int64_t BLK = 64 * GROUP_ROUNDS;
  // wave sums of both counts, then the workgroup's: the expert's first row and
  // the rows of e in the waves before this one
  auto scan = [&](int lt, int cnt, int& first, int& pos) {
    for (int o = 1; o < 64; o <<= 1) {
      lt += __shfl_xor(lt, o, 64);
      cnt += __shfl_xor(cnt, o, 64);
    }
    if (lane == 0) {
      lt_w[wv] = lt;
      m_w[wv] = cnt;
    }
    __syncthreads();
    first = 0;
    pos = 0;
    for (int w = 0; w < 16; w++) {
      first += lt_w[w];
      pos += w < wv ? m_w[w] : 0;
    }
    pos += first;
    return cnt;
  };
  int first, pos, lt = 0, cnt = 0;
  if (per <= BLK) {                                     // workgroup-uniform: one block per wave
    int v[GROUP_ROUNDS];
    group_load(ids, p0, p1, lane, v);
    group_count(v, e, lt, cnt);
    if (scan(lt, cnt, first, pos) > 0) group_place(v, e, k, p0, lane, pos, row_token, row_slot);
  } else {
    for (int64_t base = p0; base < p1; base += BLK) {
      int v[GROUP_ROUNDS];
      group_load(ids, base, p1, lane, v);
      group_count(v, e, lt, cnt);
    }
    if (scan(lt, cnt, first, pos) > 0)
      for (int64_t base = p0; base < p1; base += BLK) {
        int v[GROUP_ROUNDS];
        group_load(ids, base, p1, lane, v);
        group_place(v, e, k, base, lane, pos, row_token, row_slot);
      }
  }
  if (tid == 0) {
    offsets[e] = first;
    if (e == E - 1) offsets[E] = (int32_t)P;
  }
}

// ---------------------------------------------------------------------------
// Scale recipe, weight re-layout, tables
// ---------------------------------------------------------------------------
// Per output channel: ch = 8 * RN(amax / 448) (1 for an all-zero channel),
// s8 = e4m3(RN(s / ch)) with correctly rounded division.  Channels of at most
// 32 groups share a wave, gp lanes each (gp the smallest power of two >= G,
// the maximum an xor butterfly within the gp lanes); longer channels take one
// wave each.
inline int scales_lanes(int G) {
  int gp = 1;
  while (gp < G) gp <<= 1;
  return gp;
}
__global__ __launch_bounds__(256) void k_w4a8_scales(const uint16_t* __restrict__ sc, int64_t rows, int G,
                                                     uint8_t* __restrict__ s8, float* __restrict__ ch) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (G <= 32) {
    int gp = 1;
    while (gp < G) gp <<= 1;
    const int64_t r = wave * (64 / gp) + lane / gp;
    const int g = lane % gp;
    const bool live = r < rows && g < G;
    const float v = live ? bf16_to_f32(sc[r * G + g]) : 0.0f;
    float amax = __builtin_fabsf(v);
    for (int o = 1; o < gp; o <<= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, o, 64));
    float s = amax / 448.0f;
    if (s == 0.0f) s = 1.0f;
    const float c = 8.0f * s;
    if (live) s8[r * G + g] = (uint8_t)(e4m3_pack2<false>(clamp448(v / c), 0.0f, 0u) & 0xFFu);
    if (live && g == 0) ch[r] = c;
    return;
  }
  const int64_t r = wave;
  if (r >= rows) return;
  float amax = 0.0f;
  for (int g = lane; g < G; g += 64) amax = __builtin_fmaxf(amax, __builtin_fabsf(bf16_to_f32(sc[r * G + g])));
  for (int o = 1; o < 64; o <<= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, o, 64));
  float s = amax / 448.0f;
  if (s == 0.0f) s = 1.0f;
  const float c = 8.0f * s;
  for (int g = lane; g < G; g += 64) {
    const float v = bf16_to_f32(sc[r * G + g]) / c;
    s8[r * G + g] = (uint8_t)(e4m3_pack2<false>(clamp448(v), 0.0f, 0u) & 0xFFu);
  }
  if (lane == 0) ch[r] = c;
}

// Element 8i + j of a word moves from nibble j to nibble 2j (j < 4) or
// 2(j - 4) + 1 (j >= 4).
__device__ __forceinline__ uint32_t interleave_nibbles(uint32_t w) {
  uint32_t o = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    o |= ((w >> (4 * j)) & 0xFu) << (8 * j);
    o |= ((w >> (4 * j + 16)) & 0xFu) << (8 * j + 4);
  }
  return o;
}

__global__ __launch_bounds__(256) void k_w4a8_relayout(const uint32_t* __restrict__ in, uint32_t* out, int64_t words) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= words) return;                               // words % 4 == 0
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(in + i);
  *reinterpret_cast<u32x4_t*>(out + i) =
      u32x4_t{interleave_nibbles(v[0]), interleave_nibbles(v[1]), interleave_nibbles(v[2]), interleave_nibbles(v[3])};
}

// Byte pools of one group: lo = codes of w = 0..7, hi = codes of w = -8..-1.
struct Lut {
  uint32_t lo0, lo1, hi0, hi1;
};
__device__ __forceinline__ Lut make_lut(uint32_t s8code) {
  const float v = __builtin_amdgcn_cvt_f32_fp8((int)s8code, 0);
  uint32_t a = e4m3_pack2<false>(clamp448(v), clamp448(2.0f * v), 0u);          // P1 P2
  a = e4m3_pack2<true>(clamp448(3.0f * v), clamp448(4.0f * v), a);              // P3 P4
  uint32_t b = e4m3_pack2<false>(clamp448(5.0f * v), clamp448(6.0f * v), 0u);   // P5 P6
  b = e4m3_pack2<true>(clamp448(7.0f * v), clamp448(8.0f * v), b);              // P7 P8
  Lut L;
  L.lo0 = (a << 8) | (s8code & 0x80u);                                        // +-0 P1 P2 P3
  L.lo1 = __builtin_amdgcn_perm(b, a, 0x06050403u);                             // P4 P5 P6 P7
  L.hi0 = __builtin_amdgcn_perm(b, a, 0x04050607u) ^ 0x80808080u;               // -P8 -P7 -P6 -P5
  L.hi1 = __builtin_amdgcn_perm(b, a, 0x00010203u) ^ 0x80808080u;               // -P4 -P3 -P2 -P1
  return L;
}
// One re-laid word (8 INT4 codes) -> 8 E4M3 codes in k order.
__device__ __forceinline__ void lut_word(uint32_t w, const Lut& L, uint32_t& d0, uint32_t& d1) {
  const uint32_t se = w & 0x07070707u, so = (w >> 4) & 0x07070707u;
  const uint32_t le = __builtin_amdgcn_perm(L.lo1, L.lo0, se), he = __builtin_amdgcn_perm(L.hi1, L.hi0, se);
  const uint32_t lo = __builtin_amdgcn_perm(L.lo1, L.lo0, so), ho = __builtin_amdgcn_perm(L.hi1, L.hi0, so);
  const uint32_t me = ((w >> 1) & 0x04040404u) | 0x03020100u;                  // byte k from he if sign bit
  const uint32_t mo = ((w >> 5) & 0x04040404u) | 0x03020100u;
  d0 = __builtin_amdgcn_perm(he, le, me);
  d1 = __builtin_amdgcn_perm(ho, lo, mo);
}

// Materialised E4M3 weights (N x K codes) from re-laid words and s8.
__global__ __launch_bounds__(256) void k_w4a8_dequant(const uint32_t* __restrict__ wq, const uint8_t* __restrict__ s8,
                                                      int64_t N, int64_t K, uint8_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // word index
  const int64_t wpr = K / 8;
  if (i >= N * wpr) return;
  const int64_t n = i / wpr, k = (i % wpr) * 8;
  const Lut L = make_lut(s8[n * (K / 128) + k / 128]);
  uint32_t d0, d1;
  lut_word(wq[i], L, d0, d1);
  *reinterpret_cast<uint2*>(out + n * K + k) = uint2{d0, d1};
}

// ---------------------------------------------------------------------------
// Grouped GEMM
// ---------------------------------------------------------------------------
constexpr int MBM = 256, MBN = 256, MBK = 128;
constexpr int MA_TILE = MBM * MBK;                      // 32 KB of E4M3 rows
constexpr int MB_TILE = MBN * MBK / 2;                  // 16 KB of packed INT4
constexpr int MSTAGE = MA_TILE + MB_TILE;
constexpr int MNSTAGE = 3;                              // loads run two steps ahead
constexpr int MLDS = MNSTAGE * MSTAGE;                  // 144 KB
constexpr int MS8_CHUNK = 32;                           // groups of s8 held in LDS at a time (8 KB)
// LDS placement of the tiles' 16-byte chunks.  A ds_read_b128 serves 16
// lanes per pass over 64 banks (256 bytes), so the 16 rows one fragment read
// touches must land on distinct 16-byte bank groups.  Activation rows of 128
// bytes (two rows per 256 bytes): chunk c of row r at c ^ ((r >> 1) & 7).  W
// rows of 64 bytes (four rows per 256 bytes): chunk c of row r at
// c ^ ((r >> 2) & 3).
__device__ __forceinline__ int maswz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int mbswz(int r) { return (r >> 2) & 3; }
// The 8 waves all lie along N, each owning 256 rows x 32 channels (8 MFMA
// tiles of 32x32): every W fragment is converted through its table once per
// workgroup (with 2 x 4 waves the two M-halves converted each fragment twice),
// at twice the activation fragment reads from LDS.
constexpr int MWN = 8, MTN = MBN / MWN, MMI = MBM / 32;

__global__ __launch_bounds__(512) void k_moe_gemm(const uint8_t* __restrict__ x8, int64_t T,
                                                  const float* __restrict__ a_scale,
                                                  const int32_t* __restrict__ row_token, int64_t R,
                                                  const int32_t* __restrict__ offsets, int E, int64_t N, int64_t K,
                                                  const uint32_t* __restrict__ wq, const uint8_t* __restrict__ s8,
                                                  const float* __restrict__ ch, uint16_t* __restrict__ y,
                                                  int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int tinfo[2];
  __shared__ float rscale[MBM];                         // a_scale of each row of the tile
  __shared__ uint8_t s8l[MS8_CHUNK * MBN];              // s8 of MS8_CHUNK groups x the tile's columns
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave;
  const int l32 = lane & 31, h = lane >> 5;

  const int nwg = (int)gridDim.x;
  int pid = blockIdx.x;
  if (nwg % 8 == 0) pid = (pid % 8) * (nwg / 8) + pid / 8;
  const int tn = pid % tiles_n, mt = pid / tiles_n;

  // which expert and which of its 256-row tiles this workgroup owns
  if (wave == 0) {
    if (lane == 0) tinfo[0] = -1;
    int before = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      // the expert's rows [lo, hi), clamped to [0, R] whatever the caller's
      // offsets hold (decreasing or out-of-range offsets give empty experts)
      const int64_t lo = e < E ? (offsets[e] < 0 ? 0 : (offsets[e] > R ? R : offsets[e])) : 0;
      const int64_t hi = e < E ? (offsets[e + 1] < lo ? lo : (offsets[e + 1] > R ? R : offsets[e + 1])) : 0;
      const int cnt = (int)(hi - lo);
      const int tiles = (cnt + MBM - 1) / MBM;
      int incl = tiles;
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      const int start = before + incl - tiles;
      if (e < E && mt >= start && mt < start + tiles) {
        tinfo[0] = e;
        tinfo[1] = mt - start;
      }
      before += __shfl(incl, 63, 64);
    }
  }
  __syncthreads();
  const int e = tinfo[0];
  if (e < 0) return;                                    // whole workgroup
  const int64_t elo = offsets[e] < 0 ? 0 : (offsets[e] > R ? R : offsets[e]);
  const int64_t ehi = offsets[e + 1] < elo ? elo : (offsets[e + 1] > R ? R : offsets[e + 1]);
  const int64_t r0 = elo + (int64_t)tinfo[1] * MBM;
  const int64_t r1 = ehi < r0 + MBM ? ehi : r0 + MBM;
  const int ntile = __builtin_amdgcn_readfirstlane((int)((r1 - r0 + 31) >> 5));   // 1 .. MMI row tiles
  const int64_t n0 = (int64_t)tn * MBN;
  const int64_t rowbytes = K / 2;
  const int64_t nrows = N - n0 < MBN ? N - n0 : MBN;
  const auto ra = make_rsrc(x8, T * K);
  const auto rb = make_rsrc(reinterpret_cast<const uint8_t*>(wq) + ((int64_t)e * N + n0) * rowbytes, nrows * rowbytes);
  const int64_t G = K / 128;
  if (tid < MBM) {
    const int64_t gr = r0 + tid;
    // a gathered token index outside [0, T) reads as a zero row with scale 0
    const int64_t tok = gr < r1 ? (row_token ? (int64_t)row_token[gr] : gr) : -1;
    rscale[tid] = tok >= 0 && tok < T ? a_scale[tok] : 0.0f;
  }

  // A: 4 DMA instructions per wave, 8 gathered rows each, 16-byte chunks
  // XOR-swizzled by row; rows past the expert's end read as zeros.
  uint32_t a_off[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int r = 8 * (wave * 4 + i) + (lane >> 3);
    const int c = (lane & 7) ^ maswz(r);
    const int64_t gr = r0 + r;
    const int64_t tok = gr < r1 ? (row_token ? (int64_t)row_token[gr] : gr) : -1;
    a_off[i] = tok >= 0 && tok < T ? (uint32_t)(tok * K) + 16 * c : 0x80000000u;
  }
  // B: 2 DMA instructions per wave, 16 rows of 64 bytes each, chunks swizzled
  uint32_t b_off[2];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int r = 16 * (wave * 2 + i) + (lane >> 2);
    b_off[i] = (uint32_t)(r * rowbytes) + 16 * ((lane & 3) ^ mbswz(r));
  }
  // The step's K offset goes in the DMA's scalar offset: the per-lane offsets
  // stay in registers that nothing in the loop writes (a row past the
  // expert's end keeps its 0x80000000 offset, still past the buffer's end).
  auto issue = [&](int stage, int64_t k0) {
    uint8_t* A = lds + stage * MSTAGE;
    uint8_t* B = A + MA_TILE;
#pragma unroll
    for (int i = 0; i < 4; i++) lds_dma16(ra, A + (wave * 4 + i) * 1024, a_off[i], (uint32_t)k0);
#pragma unroll
    for (int i = 0; i < 2; i++) lds_dma16(rb, B + (wave * 2 + i) * 1024, b_off[i], (uint32_t)(k0 / 2));
  };

  // Group scales: thread t < 256 copies column n0 + t's s8 codes of groups
  // [g0, g0 + MS8_CHUNK) into s8l (group-major), so that the K loop reads them
  // from LDS and issues no loads into registers (which would wait on the
  // tile loads queued ahead of them).
  const int myc = wn * MTN + l32;
  auto load_s8_chunk = [&](int g0) {
    if (tid < MBN) {
      int64_t c = n0 + tid;
      c = c < N ? c : N - 1;
      const uint8_t* p = s8 + ((int64_t)e * N + c) * G + g0;
      const int cnt = (int)(G - g0) < MS8_CHUNK ? (int)(G - g0) : MS8_CHUNK;
      if (G % 4 == 0) {                                 // 4-byte aligned rows: dword loads
        const uint32_t* p4 = reinterpret_cast<const uint32_t*>(p);
        uint32_t v[MS8_CHUNK / 4];
#pragma unroll
        for (int q = 0; q < MS8_CHUNK / 4; q++) v[q] = 4 * q < cnt ? p4[q] : 0u;
#pragma unroll
        for (int q = 0; q < MS8_CHUNK / 4; q++)
          if (4 * q < cnt)
#pragma unroll
            for (int b = 0; b < 4; b++) s8l[(4 * q + b) * MBN + tid] = (uint8_t)(v[q] >> (8 * b));
      } else {
        uint8_t v[MS8_CHUNK];
#pragma unroll
        for (int q = 0; q < MS8_CHUNK; q++) v[q] = p[q < cnt ? q : cnt - 1];   // entries past G: unused
#pragma unroll
        for (int q = 0; q < MS8_CHUNK; q++) s8l[q * MBN + tid] = v[q];
      }
    }
  };
  // raw s8 of step k (its chunk resident)
  auto s8_of = [&](int k) -> uint32_t { return s8l[(k % MS8_CHUNK) * MBN + myc]; };

  f32x16_t acc[MMI];
#pragma unroll
  for (int i = 0; i < MMI; i++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[i][r] = 0.0f;

  // B operand of half s2 of a step (K 64): 32 E4M3 codes of the lane's column
  auto lut_half = [&](const uint8_t* B, int s2, const Lut& L, i32x8_t& bf) {
    const int br = wn * MTN + l32;
    const u32x4_t pw = ld16(B + br * 64 + 16 * ((2 * s2 + h) ^ mbswz(br)));
    uint32_t d[8];
#pragma unroll
    for (int q = 0; q < 4; q++) lut_word(pw[q], L, d[2 * q], d[2 * q + 1]);
    bf = i32x8_t{(int)d[0], (int)d[1], (int)d[2], (int)d[3], (int)d[4], (int)d[5], (int)d[6], (int)d[7]};
  };
  // A operand of row tile i and half s2 of the step in stage A
  auto load_a = [&](const uint8_t* A, int s2, int i) -> i32x8_t {
    const int r = 32 * i + l32;
    const int c0 = 4 * s2 + 2 * h;
    const u32x4_t p0 = ld16(A + r * 128 + ((c0 ^ maswz(r)) << 4));
    const u32x4_t p1 = ld16(A + r * 128 + (((c0 + 1) ^ maswz(r)) << 4));
    return i32x8_t{(int)p0[0], (int)p0[1], (int)p0[2], (int)p0[3], (int)p1[0], (int)p1[1], (int)p1[2], (int)p1[3]};
  };
  // the MFMAs of half s2 over the first NT row tiles (NT is a compile-time
  // count, so the unrolled MFMA sequence stays free of branches); tile i + 1's
  // operand is read while tile i's MFMA runs
  auto mfma_half = [&](auto nt, const uint8_t* A, int s2, const i32x8_t& bf) {
    constexpr int NT = decltype(nt)::value;
    i32x8_t an = load_a(A, s2, 0);
#pragma unroll
    for (int i = 0; i < NT; i++) {
      const i32x8_t af = an;
      if (i + 1 < NT) an = load_a(A, s2, i + 1);
      acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, acc[i], 0, 0, 0, 127, 0, 127);
    }
  };

  // Software pipeline.  Step k's loads (group k) go to stage k % 3, two steps
  // ahead.  At the top of step k groups <= k + 1 are resident and visible; the
  // MFMAs of each half run on operands converted during the previous half, so
  // the table lookups of one half overlap the matrix work of the other: half 0
  // converts half 1 of step k, half 1 converts half 0 of step k + 1.  The
  // barrier at the end of step k publishes group k + 2 and retires every read
  // of stage k % 3, which step k + 1 then refills with group k + 3.
  const int nk = (int)(K / MBK);
  issue(0, 0);
  if (nk > 1) issue(1, MBK);
  load_s8_chunk(0);
  wait_vm<0>();
  __syncthreads();                                      // also publishes rscale and s8l
  Lut Lc = make_lut(s8_of(0));
  i32x8_t bc, bn;
  lut_half(lds + MA_TILE, 0, Lc, bc);

  // The last row tile of an expert is usually partial: the K loop runs the
  // MFMAs of the first 2, 4, 6 or 8 row tiles (the fewest that cover the
  // tile's rows), one instance of the loop per count.
  auto k_loop = [&](auto nt, auto reload) {
    int stage = 0;
    for (int kt = 0; kt < nk; kt++) {
      const int st1 = stage == 2 ? 0 : stage + 1;
      const int st2 = st1 == 2 ? 0 : st1 + 1;
      // K > MS8_CHUNK groups: the next chunk of s8 replaces the current one
      // before step kt's look-ahead reads it (the last read of the current
      // chunk was in step kt - 1, before its closing barrier)
      if constexpr (decltype(reload)::value) {
        if ((kt + 1) % MS8_CHUNK == 0 && kt + 1 < nk) {
          load_s8_chunk(kt + 1);
          __syncthreads();
        }
      }
      if (kt + 2 < nk) issue(st2, (int64_t)(kt + 2) * MBK);
      // (on the last step the second conversion reads a stale stage; unused)
      const uint8_t* A = lds + stage * MSTAGE;
      lut_half(A + MA_TILE, 1, Lc, bn);
      mfma_half(nt, A, 0, bc);
      Lc = make_lut(s8_of(kt + 1 < nk ? kt + 1 : kt));
      lut_half(lds + st1 * MSTAGE + MA_TILE, 0, Lc, bc);
      mfma_half(nt, A, 1, bn);
      wait_vm<0>();
      tile_barrier();
      stage = st1;
    }
  };
  auto by_rows = [&](auto reload) {
    if (ntile > 6) k_loop(std::integral_constant<int, 8>{}, reload);
    else if (ntile > 4) k_loop(std::integral_constant<int, 6>{}, reload);
    else if (ntile > 2) k_loop(std::integral_constant<int, 4>{}, reload);
    else k_loop(std::integral_constant<int, 2>{}, reload);
  };
  if (G <= MS8_CHUNK) by_rows(std::false_type{});
  else k_loop(std::integral_constant<int, MMI>{}, std::true_type{});   // K > 4096: every row tile

  // epilogue: C element r of a 32x32 tile sits at row 8*(r/4) + 4*h + r%4, col l32.
  // Stores go through a buffer range covering the tile's valid rows, so rows
  // past the expert's end are dropped by the hardware and offsets stay 32-bit.
  const auto ry = make_rsrc(y + r0 * N, (r1 - r0) * N * 2);
  const uint32_t rowb = (uint32_t)(N * 2);
  const int64_t col = n0 + wn * MTN + l32;
  const float cs = col < N ? ch[(int64_t)e * N + col] : 0.0f;
  const uint32_t cb = col < N ? (uint32_t)(col * 2) : 0x80000000u;   // columns past N: out of range
#pragma unroll
  for (int i = 0; i < MMI; i++) {
    if (i >= ntile) break;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int lr = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
      const uint32_t v = f32_to_bf16_bits(acc[i][r] * (rscale[lr] * cs));
      __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, ry, (int)((uint32_t)lr * rowb + cb), 0, 0);
    }
  }
}

}  // namespace

extern "C" {

wq_status wq_moe_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids, float* weights,
                       int32_t* offsets, int32_t* row_token, int32_t* row_slot, void* stream) {
  if (T < 0 || E < 1 || E > 64 || k < 1 || k > E) return WQ_EINVAL;
  if (T * k > 0x7FFFFFFFLL) return WQ_EINVAL;
  if (!offsets || (T > 0 && (!logits || !ids || !weights || !row_token || !row_slot))) return WQ_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (T > 0) k_route<<<(unsigned)((T + 3) / 4), 256, 0, s>>>(logits, T, E, k, ids, weights);
  k_group<<<(unsigned)E, 1024, 0, s>>>(ids, T, E, k, offsets, row_token, row_slot);
  return wq_launch_status();
}

wq_status wq_w4a8_prepack(const uint32_t* wq, const uint16_t* scales, int64_t experts, int64_t N, int64_t K,
                          uint32_t* wq_out, uint8_t* s8, float* ch, void* stream) {
  if (experts < 1 || N < 1 || K < 128 || K % 128) return WQ_EINVAL;
  if (!wq || !scales || !wq_out || !s8 || !ch) return WQ_EINVAL;
  if (!wq_aligned(wq) || !wq_aligned(wq_out)) return WQ_EALIGN;
  if (!wq_numel_ok(experts * N, K)) return WQ_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const int64_t rows = experts * N, G = K / 128, words = rows * (K / 8);
  const int64_t scale_waves = G <= 32 ? (rows + 64 / scales_lanes((int)G) - 1) / (64 / scales_lanes((int)G)) : rows;
  k_w4a8_scales<<<(unsigned)((scale_waves + 3) / 4), 256, 0, s>>>(scales, rows, (int)G, s8, ch);
  k_w4a8_relayout<<<(unsigned)((words / 4 + 255) / 256), 256, 0, s>>>(wq, wq_out, words);
  return wq_launch_status();
}

wq_status wq_w4a8_dequant(const uint32_t* wq, const uint8_t* s8, int64_t N, int64_t K, uint8_t* codes, void* stream) {
  if (N < 1 || K < 128 || K % 128 || !wq || !s8 || !codes) return WQ_EINVAL;
  if (!wq_numel_ok(N, K)) return WQ_EINVAL;
  const int64_t words = N * (K / 8);
  k_w4a8_dequant<<<(unsigned)((words + 255) / 256), 256, 0, (hipStream_t)stream>>>(wq, s8, N, K, codes);
  return wq_launch_status();
}

wq_status wq_moe_gemm_w4a8(const uint8_t* x8, int64_t T, const float* a_scale, const int32_t* row_token, int64_t R,
                           const int32_t* offsets, int32_t experts, int64_t N, int64_t K, const uint32_t* wq,
                           const uint8_t* s8, const float* ch, uint16_t* y, void* stream) {
  if (T < 1 || R < 0 || experts < 1 || N < 1 || K < 128 || K % 128) return WQ_EINVAL;
  if (!x8 || !a_scale || !offsets || !wq || !s8 || !ch || (R > 0 && !y)) return WQ_EINVAL;
  if (!row_token && R != T) return WQ_EINVAL;
  if (!wq_aligned(x8) || !wq_aligned(wq)) return WQ_EALIGN;
  // 32-bit buffer offsets: the activations, one expert's 256-row W panel, one
  // 256-row output tile
  if (T * K > 0x7FFFFFF0LL || (int64_t)MBN * K / 2 > 0x7FFFFFF0LL || (int64_t)MBM * N * 2 > 0x7FFFFFF0LL ||
      R > 0x7FFFFFFFLL)
    return WQ_EINVAL;
  if (R == 0) return WQ_OK;
  static bool done[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return WQ_EHIP;
  if (dev < 0 || dev >= 64 || !done[dev]) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(k_moe_gemm), hipFuncAttributeMaxDynamicSharedMemorySize,
                            MLDS) != hipSuccess)
      return WQ_EHIP;
    if (dev >= 0 && dev < 64) done[dev] = true;
  }
  const int64_t tiles_m = (R + MBM - 1) / MBM + experts;   // each expert adds at most one partial tile
  const int64_t tiles_n = (N + MBN - 1) / MBN;
  if (tiles_m * tiles_n > 0x7FFFFFFFLL) return WQ_EINVAL;
  k_moe_gemm<<<(unsigned)(tiles_m * tiles_n), 512, MLDS, (hipStream_t)stream>>>(
      x8, T, a_scale, row_token, R, offsets, experts, N, K, wq, s8, ch, y, (int)tiles_n);
  return wq_launch_status();
}

}  // extern "C"
