// Compact block metadata: the uint8 in-block positions of the pruning pass
// to and from packed per-block codes.
//
// A block's kept positions c_1 < ... < c_n (of m) become either
//  - a combinatorial code of ceil(log2 C(m, n)) bits: the rank of the set in
//    colexicographic order, sum_i C(c_i, i) (the activation sparsification
//    guide's s2.1 table counts C(m, n) patterns per block and s4.1 stores a
//    2:4 block in 3 bits), or
//  - an m-bit mask, bit j set when position j is kept.
// Codes are laid end to end along a token row, block 0 in the lowest bits,
// least significant bit first, in 32-bit words; every row starts on a fresh
// word.  Both kernels are bound by HBM: one thread per block, 256 blocks per
// workgroup, and a wave's 64 codes fill exactly 2 x width whole words, which
// the wave assembles in LDS and stores with one coalesced write.  2:4 codes
// and masks of rows that fill whole words take a flat-stream pair of kernels
// instead (k_encode24_flat, k_decode24_flat below).
#include "spa_common.h"
#include "spa_launch.h"

namespace spa {

// Binomial coefficients C(a, b), 0 <= a, b <= 32 (C(32, 16) = 601080390 fits
// in 32 bits), from Pascal's rule at compile time.
struct Binom {
  uint32_t c[33][33];
};
constexpr Binom make_binom() {
  Binom t{};
  for (int a = 0; a <= 32; ++a) {
    t.c[a][0] = 1;
    for (int b = 1; b <= a; ++b) t.c[a][b] = t.c[a - 1][b - 1] + (b <= a - 1 ? t.c[a - 1][b] : 0u);
  }
  return t;
}
__constant__ Binom kBinom = make_binom();

// Bits per block: m for the mask; ceil(log2 C(m, n)) for the code (0 when n == m).
int meta_width(int n, int m, int format) {
  if (format == SPA_META_BITMAP) return m;
  const uint32_t count = make_binom().c[m][n];
  int w = 0;
  while (w < 32 && (uint64_t(1) << w) < count) ++w;
  return w;
}

struct MetaArgs {
  const uint8_t* idx;   // encode input [t][nb * n]
  uint8_t* idx_out;     // decode output [t][nb * n]
  uint32_t* codes;      // [t][row_words]
  int nb;               // blocks per row
  int chunks;           // workgroups per row
  int n, m, width, row_words, format;
  int aligned;          // rows of positions start on 16-byte boundaries
};

// Blocks per thread: 16 bytes of positions (one vector access) when n
// divides 16, else one block with byte accesses.
template <int NV>
constexpr int blocks_per_thread() { return NV ? 16 / NV : 1; }

// Positions of blocks b .. b + BT - 1 of one row; blocks past the row read 0.
template <int NV, int BT>
__device__ __forceinline__ void load_group(const uint8_t* row, int b, const MetaArgs& a, uint8_t (&c)[BT * NV]) {
  if (a.aligned && b + BT <= a.nb) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + (size_t)b * NV);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 16; ++j) c[j] = (uint8_t)(w[j >> 2] >> (8 * (j & 3)));
  } else {
#pragma unroll
    for (int j = 0; j < BT * NV; ++j) c[j] = b + j / NV < a.nb ? row[(size_t)b * NV + j] : (uint8_t)0;
  }
}

template <int NV, int BT>
__device__ __forceinline__ void store_group(uint8_t* row, int b, const MetaArgs& a, const uint8_t (&c)[BT * NV]) {
  if (a.aligned && b + BT <= a.nb) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = (uint32_t)c[4 * q] | ((uint32_t)c[4 * q + 1] << 8) | ((uint32_t)c[4 * q + 2] << 16) |
             ((uint32_t)c[4 * q + 3] << 24);
    *reinterpret_cast<uint4*>(row + (size_t)b * NV) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
#pragma unroll
    for (int j = 0; j < BT * NV; ++j)
      if (b + j / NV < a.nb) row[(size_t)b * NV + j] = c[j];
  }
}

// The rows C(., i), i = 0..n, of the binomial table into LDS as tab[i][c].
__device__ __forceinline__ void load_tab(uint32_t (*tab)[33], int n) {
  for (int e = threadIdx.x; e < (n + 1) * 33; e += blockDim.x) {
    const int i = e / 33, c = e - i * 33;
    tab[i][c] = kBinom.c[c][i];
  }
}

// One block's code from its positions (an input position >= 32 is folded into
// range: the code is then unspecified, the table access stays in bounds).
__device__ __forceinline__ uint32_t add_pos(uint32_t code, uint32_t c, int j, int format,
                                            const uint32_t (*tab)[33]) {
  c &= 31u;
  return code + (format == SPA_META_BITMAP ? (1u << c) : tab[j + 1][c]);
}

// Work split: a thread takes G groups of BT consecutive blocks (16 bytes of
// positions per group); group s of lane l in wave v starts at block
// (((chunk * 4 + v) * G + s) * 64 + l) * BT of its row, so each load is
// coalesced across the wave.  A wave's codes fill 2 * G * BT * width whole
// words, assembled in LDS (bitwise OR, as a code may straddle two words) and
// stored coalesced.  G = 1: token rows are short (a 2:4 row of 16384
// channels is 8 KB of positions), and larger groups left lanes idle (4
// groups: 16 -> 27 us for the 2:4 encode at 4096 x 16384).
template <int NV>
constexpr int groups_per_thread() { return 1; }

// C24: 2:4 combinatorial codes, formed and read without the table.
template <int NV, bool C24>
__global__ void __launch_bounds__(256) k_encode_meta(MetaArgs a) {
  constexpr int BT = blocks_per_thread<NV>(), G = groups_per_thread<NV>();
  extern __shared__ uint32_t s_dyn[];
  __shared__ uint32_t s_binom[33][33];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int row = blockIdx.x / a.chunks;
  const int chunk = blockIdx.x - row * a.chunks;
  const int w = a.width;
  const int nw = 2 * G * BT * w;                           // words of this wave
  uint32_t* s_words = s_dyn + wv * nw;
  const int64_t wb = (int64_t)(chunk * 4 + wv) * G * 64 * BT;   // the wave's first block
  // 2:4 codes need no table: C(lo, 1) + C(hi, 2) = lo + hi (hi - 1) / 2
  if (a.format == SPA_META_COMB && !C24) load_tab(s_binom, NV ? NV : a.n);
  for (int j = lane; j < nw; j += 64) s_words[j] = 0u;

  const uint8_t* rp = a.idx + (size_t)row * a.nb * (NV ? NV : a.n);
  uint32_t code[G][BT];
  if constexpr (NV > 0) {
    uint8_t c[G][BT * NV];
#pragma unroll
    for (int g = 0; g < G; ++g) load_group<NV, BT>(rp, (int)(wb + (g * 64 + lane) * BT), a, c[g]);
    __syncthreads();                                       // the table and the cleared words
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int b = (int)(wb + (g * 64 + lane) * BT);
#pragma unroll
      for (int q = 0; q < BT; ++q) {
        uint32_t v = 0;
        if constexpr (C24) {
          const uint32_t lo = c[g][q * NV] & 31u, hi = c[g][q * NV + NV - 1] & 31u;
          v = lo + hi * (hi - 1u) / 2u;
        } else {
#pragma unroll
          for (int jj = 0; jj < NV; ++jj) v = add_pos(v, c[g][q * NV + jj], jj, a.format, s_binom);
        }
        code[g][q] = b + q < a.nb ? v : 0u;
      }
    }
  } else {
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int b = (int)(wb + g * 64 + lane);
      uint32_t v = 0;
      if (b < a.nb)
        for (int jj = 0; jj < a.n; ++jj) v = add_pos(v, rp[(size_t)b * a.n + jj], jj, a.format, s_binom);
      code[g][0] = v;
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int q = 0; q < BT; ++q) {
      const int bit = ((g * 64 + lane) * BT + q) * w;
      if (code[g][q]) {
        atomicOr(&s_words[bit >> 5], code[g][q] << (bit & 31));
        if ((bit & 31) + w > 32) atomicOr(&s_words[(bit >> 5) + 1], code[g][q] >> (32 - (bit & 31)));
      }
    }
  __syncthreads();
  const int64_t gbase = (wb * w) >> 5;                     // wb * w is a multiple of 64
  uint32_t* out = a.codes + (size_t)row * a.row_words;
  for (int j = lane; j < nw; j += 64)
    if (gbase + j < a.row_words) out[gbase + j] = s_words[j];
}

template <int NV, bool C24>
__global__ void __launch_bounds__(256) k_decode_meta(MetaArgs a) {
  constexpr int BT = blocks_per_thread<NV>(), G = groups_per_thread<NV>();
  constexpr int CAP = NV ? NV : 32;                        // positions per block held in registers
  extern __shared__ uint32_t s_dyn[];
  __shared__ uint32_t s_binom[33][33];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int row = blockIdx.x / a.chunks;
  const int chunk = blockIdx.x - row * a.chunks;
  const int w = a.width, m = a.m;
  const int n = NV ? NV : a.n;
  const int nw = 2 * G * BT * w;
  uint32_t* s_words = s_dyn + wv * nw;
  const int64_t wb = (int64_t)(chunk * 4 + wv) * G * 64 * BT;
  // 2:4 codes 0..5 name the pairs {0,1}, {0,2}, {1,2}, {0,3}, {1,3}, {2,3}
  // (colex order): nibble `code` of kPairs24 holds lo | hi << 2; the unused
  // codes 6 and 7 give {2,3}, as the greedy unranking below does
  constexpr uint32_t kPairs24 = 0xEEEDC984u;
  if (a.format == SPA_META_COMB && !C24) load_tab(s_binom, n);
  {
    const int64_t gbase = (wb * w) >> 5;
    const uint32_t* in = a.codes + (size_t)row * a.row_words;
    for (int j = lane; j < nw; j += 64) s_words[j] = gbase + j < a.row_words ? in[gbase + j] : 0u;
  }
  __syncthreads();

  uint8_t* rp = a.idx_out + (size_t)row * a.nb * n;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    uint8_t c[BT * CAP];
#pragma unroll
    for (int q = 0; q < BT; ++q) {
      uint32_t code = 0;
      if (w > 0) {
        const int bit = ((g * 64 + lane) * BT + q) * w, sh = bit & 31;
        uint64_t v = s_words[bit >> 5];
        if (sh + w > 32) v |= (uint64_t)s_words[(bit >> 5) + 1] << 32;
        code = (uint32_t)((v >> sh) & ((uint64_t(1) << w) - 1));
      }
      uint32_t mask = code;
      if constexpr (C24) {
        const uint32_t pr = (kPairs24 >> (4u * code)) & 15u;    // code < 8 (3 bits)
        mask = (1u << (pr & 3u)) | (1u << (pr >> 2));
      } else if (a.format == SPA_META_COMB) {
        // greedy unranking in one pass over the positions, largest first: take
        // c while i positions remain and C(c, i) <= the remaining rank (C(c, i)
        // is 0 once c < i, so exactly n are taken); the same m steps on every
        // lane
        uint32_t r = code;
        int i = n;
        mask = 0;
        for (int cc = m - 1; cc >= 0; --cc) {
          const uint32_t bin = s_binom[i][cc];
          const bool take = i > 0 && bin <= r;
          mask |= take ? (1u << cc) : 0u;
          r -= take ? bin : 0u;
          i -= take ? 1 : 0;
        }
      }
      // the set bits in ascending order; a mask without n set bits gives
      // unspecified positions (zeros), never an access out of bounds
#pragma unroll
      for (int s2 = 0; s2 < CAP; ++s2) {
        c[q * CAP + s2] = (uint8_t)(mask ? __builtin_ctz(mask) : 0);
        mask &= mask - 1u;
      }
    }
    if constexpr (NV > 0) {
      store_group<NV, BT>(rp, (int)(wb + (g * 64 + lane) * BT), a, c);
    } else {
      const int b = (int)(wb + g * 64 + lane);
      if (b < a.nb) {
#pragma unroll
        for (int s2 = 0; s2 < CAP; ++s2)
          if (s2 < n) rp[(size_t)b * n + s2] = c[s2];
      }
    }
  }
}

// 2:4 combinatorial codes of rows whose codes fill whole words (blocks per
// row a multiple of 32): 32 blocks are 64 bytes of positions and exactly three
// code words, so over all rows the positions and the codes are each one flat
// stream.  Lanes 4u .. 4u + 3 share unit u of 32 blocks: lane 4u + r holds
// blocks 8r .. 8r + 7 (one 16-byte piece of positions, loaded coalesced) and
// their 24 code bits, bits 24r .. 24r + 23 of the unit's 96.  Code word r is
// then lane r's bits from 8r up and lane r + 1's below (encode), and lane r's
// piece is its word from 8r down and lane r - 1's word above (decode): one
// in-quad move each way, no LDS and no barrier.  Each thread takes kFlatG
// pieces, all loads in flight first.
constexpr int kFlatG = 4;

__device__ __forceinline__ uint32_t quad_next(uint32_t v) {    // lane r + 1 of the quad (lane 3: itself)
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xF9, 0xF, 0xF, false);   // quad_perm [1,2,3,3]
}
__device__ __forceinline__ uint32_t quad_prev(uint32_t v) {    // lane r - 1 of the quad (lane 0: itself)
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x90, 0xF, 0xF, false);   // quad_perm [0,0,1,2]
}

// pieces: 16-byte pieces of positions over all rows (four per unit).  With
// BITMAP (4-bit masks, blocks per row a multiple of 8) a piece's eight blocks
// are exactly one code word: lane p stores word p, and no lanes are shared.
template <bool BITMAP>
__global__ void __launch_bounds__(256) k_encode24_flat(const uint4* __restrict__ pos, uint32_t* __restrict__ codes,
                                                        int64_t pieces) {
  const int64_t stride = (int64_t)gridDim.x * 256, p0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const uint32_t r = threadIdx.x & 3u;
  uint4 v[kFlatG];
#pragma unroll
  for (int g = 0; g < kFlatG; ++g) {
    const int64_t p = p0 + g * stride;
    v[g] = p < pieces ? pos[p] : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int g = 0; g < kFlatG; ++g) {
    const int64_t p = p0 + g * stride;                     // p % 4 == r: a unit's lanes are all in or all out
    const uint32_t d[4] = {v[g].x, v[g].y, v[g].z, v[g].w};
    uint32_t bits = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // block e: positions lo, hi in bytes 2e, 2e + 1; C(lo, 1) + C(hi, 2), held
      // to its 3 bits (positions past the block give an unspecified code only)
      const uint32_t lo = (d[e >> 1] >> (16 * (e & 1))) & 31u, hi = (d[e >> 1] >> (16 * (e & 1) + 8)) & 31u;
      if constexpr (BITMAP) bits |= (((1u << lo) | (1u << hi)) & 15u) << (4 * e);
      else bits |= ((lo + hi * (hi - 1u) / 2u) & 7u) << (3 * e);
    }
    if constexpr (BITMAP) {
      if (p < pieces) codes[p] = bits;
    } else {
      const uint32_t next = quad_next(bits);
      if (p < pieces && r < 3u) codes[(p >> 2) * 3 + r] = (bits >> (8u * r)) | (next << (24u - 8u * r));
    }
  }
}

template <bool BITMAP>
__global__ void __launch_bounds__(256) k_decode24_flat(const uint32_t* __restrict__ codes, uint4* __restrict__ pos,
                                                        int64_t pieces) {
  // 2:4 codes 0..5 name the pairs {0,1}, {0,2}, {1,2}, {0,3}, {1,3}, {2,3};
  // nibble `code` of kPairs holds lo | hi << 2 (6 and 7 give {2,3})
  constexpr uint32_t kPairs = 0xEEEDC984u;
  const int64_t stride = (int64_t)gridDim.x * 256, p0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const uint32_t r = threadIdx.x & 3u;
  uint32_t own[kFlatG];
#pragma unroll
  for (int g = 0; g < kFlatG; ++g) {
    const int64_t p = p0 + g * stride;
    if constexpr (BITMAP) own[g] = p < pieces ? codes[p] : 0u;
    else own[g] = p < pieces ? codes[(p >> 2) * 3 + (r < 3u ? r : 2u)] : 0u;   // lane 3 reads word 2 as lane 2
  }
#pragma unroll
  for (int g = 0; g < kFlatG; ++g) {
    const int64_t p = p0 + g * stride;
    uint32_t bits = own[g];
    if constexpr (!BITMAP) {
      const uint32_t prev = quad_prev(own[g]);
      bits = r == 0u ? own[g] : r == 3u ? own[g] >> 8 : (prev >> (32u - 8u * r)) | (own[g] << (8u * r));
    }
    uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t lo, hi;
      if constexpr (BITMAP) {
        // the two lowest set bits (a mask without two gives zeros, below m)
        uint32_t mk = (bits >> (4 * e)) & 15u;
        lo = mk ? (uint32_t)__builtin_ctz(mk) : 0u;
        mk &= mk - 1u;
        hi = mk ? (uint32_t)__builtin_ctz(mk) : 0u;
      } else {
        const uint32_t pr = (kPairs >> (4u * ((bits >> (3 * e)) & 7u))) & 15u;
        lo = pr & 3u;
        hi = pr >> 2;
      }
      d[e >> 1] |= (lo | (hi << 8)) << (16 * (e & 1));
    }
    if (p < pieces) pos[p] = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

template <bool ENCODE>
static hipError_t meta_launch(const MetaArgs& a, int t, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)a.chunks * t));
#define SPA_META_CASE(NV)                                                                            \
  {                                                                                                  \
    const size_t lds = (size_t)4 * 2 * groups_per_thread<NV>() * blocks_per_thread<NV>() * a.width * 4; \
    if (ENCODE) hipLaunchKernelGGL((k_encode_meta<NV, false>), grid, dim3(256), lds, st, a);         \
    else hipLaunchKernelGGL((k_decode_meta<NV, false>), grid, dim3(256), lds, st, a);                \
  }                                                                                                  \
  break;
  if (a.n == 2 && a.m == 4 && a.format == SPA_META_COMB) {
    const size_t lds = (size_t)4 * 2 * groups_per_thread<2>() * blocks_per_thread<2>() * a.width * 4;
    if (ENCODE) hipLaunchKernelGGL((k_encode_meta<2, true>), grid, dim3(256), lds, st, a);
    else hipLaunchKernelGGL((k_decode_meta<2, true>), grid, dim3(256), lds, st, a);
    return hipGetLastError();
  }
  switch (a.n) {
    case 1: SPA_META_CASE(1)
    case 2: SPA_META_CASE(2)
    case 4: SPA_META_CASE(4)
    case 8: SPA_META_CASE(8)
    case 16: SPA_META_CASE(16)
    default: SPA_META_CASE(0)
  }
#undef SPA_META_CASE
  return hipGetLastError();
}

hipError_t launch_meta(bool encode, const uint8_t* idx, uint8_t* idx_out, uint32_t* codes, int t, int k, int n,
                       int m, int format, hipStream_t st) {
  MetaArgs a{};
  a.idx = idx;
  a.idx_out = idx_out;
  a.codes = codes;
  a.nb = k / m;
  a.n = n;
  a.m = m;
  a.format = format;
  a.width = meta_width(n, m, format);
  a.row_words = (int)(((int64_t)a.nb * a.width + 31) / 32);
  // blocks per workgroup: 256 threads x G groups (1) x BT blocks
  const int bt = (n == 1 || n == 2 || n == 4 || n == 8 || n == 16) ? 16 / n : 1;
  a.chunks = (int)(((int64_t)a.nb + 256 * bt - 1) / (256 * bt));
  a.aligned = ((int64_t)a.nb * n) % 16 == 0;
  if (t == 0 || a.nb == 0) return hipSuccess;
  if ((int64_t)a.chunks * t > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (encode && a.row_words == 0) return hipSuccess;      // nothing to store
  const bool bitmap = format == SPA_META_BITMAP;
  if (n == 2 && m == 4 && a.nb % (bitmap ? 8 : 32) == 0) {
    const int64_t pieces = (int64_t)t * a.nb / 8;          // 16 bytes of positions = 8 blocks
    const int64_t grid = (pieces + 256 * kFlatG - 1) / (256 * kFlatG);
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const dim3 g((unsigned)grid);
    const uint4* in = reinterpret_cast<const uint4*>(idx);
    uint4* out = reinterpret_cast<uint4*>(idx_out);
    if (encode && bitmap) hipLaunchKernelGGL(k_encode24_flat<true>, g, dim3(256), 0, st, in, codes, pieces);
    else if (encode) hipLaunchKernelGGL(k_encode24_flat<false>, g, dim3(256), 0, st, in, codes, pieces);
    else if (bitmap) hipLaunchKernelGGL(k_decode24_flat<true>, g, dim3(256), 0, st, codes, out, pieces);
    else hipLaunchKernelGGL(k_decode24_flat<false>, g, dim3(256), 0, st, codes, out, pieces);
    return hipGetLastError();
  }
  return encode ? meta_launch<true>(a, t, st) : meta_launch<false>(a, t, st);
}

}  // namespace spa
