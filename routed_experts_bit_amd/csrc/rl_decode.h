// Decode of the Q2B and T1 expert blocks (host + device code, so the same routine is
// exercised by a CPU unit test and runs inside the gfx950 kernels).
//
// The matrix kernels never materialise decoded weights in memory (Red Lite dev75, "Prompt
// ingestion": dequantising whole experts per chunk would write gigabytes per layer).  Each
// lane decodes a strip of consecutive values of one weight row straight into MFMA operands,
// 8 values per operand.  An operand holds the exact small integer s*c (|s*c| <= 45 for Q2B,
// <= 7 for T1) as bf16 or fp16, both exact; the fp16 block scale d is applied to the fp32
// accumulator once per 256-value block.  Strips start at multiples of 8, so an operand never
// straddles a sub-scale boundary (16 values for Q2B, 32 for T1).
//
// Two small tables (built once per work-group in LDS) carry the bit work:
//   tern[b]     T1 byte b (0..242) -> its five base-3 digits, least significant first, as
//               2-bit fields (10 bits); bytes 243..255 map to five 1-digits (value 0)
//   val[s][q]   scale s, 8-bit quad q of four 2-bit codes -> the four operands s*c as 16-bit
//               floats (64 bits).  T1: c = digit - 1 (s < 8); Q2B: c = 2q - 3 (s < 16)
// A T1 strip first turns its (up to 14) digit bytes into one 2-bit digit stream through
// `tern`, shifted so that the strip's first value is digit 0; the stream (and a Q2B strip's
// code bytes directly) is then read 8 bits = 4 values at a time through `val`.
//
// A strip is handled in two phases so that kernels can issue the loads of the next block
// long before decoding it: StripRaw::load issues aligned dword loads only (block header and
// the strip's byte window), Strip::prepare turns them into code words, Strip::frag returns
// operands.  Loads never touch a dword that holds no byte of the matrix: reads go through a
// source whose device form is a buffer resource over the matrix (out-of-range dwords read 0).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

namespace rl {

constexpr int QT_Q2B = 1;
constexpr int QT_T1 = 2;

template <int QT>
struct Fmt;
template <>
struct Fmt<QT_Q2B> {
    static constexpr int BYTES = 74;
    static constexpr int NSCALE = 16;
    static constexpr int HDR_DW = 4;  // bytes 0..9 of a block at any alignment
};
template <>
struct Fmt<QT_T1> {
    static constexpr int BYTES = 57;
    static constexpr int NSCALE = 8;
    static constexpr int HDR_DW = 2;  // bytes 0..4 of a block at any alignment
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

// ------------------------------------------------------------------ scalar helpers
__host__ __device__ inline float half_bits_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// 16-bit float pattern of a small integer (|v| <= 45): exact in both bf16 and fp16.
template <bool F16>
__host__ __device__ constexpr uint32_t int_to_op16(int v) {
    float f = (float)v;
    if constexpr (F16) {
        return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
    } else {
        return __builtin_bit_cast(uint32_t, f) >> 16;  // low 16 bits are zero for these values
    }
}

__host__ __device__ inline uint32_t funnel(uint32_t hi, uint32_t lo, uint32_t bytes) {
    return (uint32_t)((((uint64_t)hi << 32) | lo) >> (8 * bytes));
}

// Bytes of `tbl` picked by the four selector bytes of `sel` (each 0..3).
__host__ __device__ inline uint32_t byte_select(uint32_t tbl, uint32_t sel) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_perm(0u, tbl, sel);
#else
    uint32_t r = 0;
    for (int b = 0; b < 4; ++b) r |= ((tbl >> (8 * ((sel >> (8 * b)) & 3u))) & 255u) << (8 * b);
    return r;
#endif
}

// Bytes of the pair (hi:lo) picked by the four selector bytes of `sel` (0..3 from lo, 4..7 from hi).
__host__ __device__ inline uint32_t perm2(uint32_t hi, uint32_t lo, uint32_t sel) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_perm(hi, lo, sel);
#else
    const uint64_t v = ((uint64_t)hi << 32) | lo;
    uint32_t r = 0;
    for (int b = 0; b < 4; ++b) r |= (uint32_t)((v >> (8 * ((sel >> (8 * b)) & 7u))) & 255u) << (8 * b);
    return r;
#endif
}

// ------------------------------------------------------------------ tables
__host__ __device__ constexpr uint32_t tern_entry(uint32_t b) {
    if (b > 242) return 0x155u;  // five 1-digits
    uint32_t r = 0;
    for (int i = 0; i < 5; ++i) {
        uint32_t q = b / 3u;
        r |= (b - 3u * q) << (2 * i);
        b = q;
    }
    return r;
}

// Entry `idx` = s*256 + q of the value table.
template <int QT, bool F16>
__host__ __device__ constexpr uint64_t val_entry(int idx) {
    const int s = idx >> 8, q = idx & 255;
    uint64_t r = 0;
    for (int i = 0; i < 4; ++i) {
        int c = (q >> (2 * i)) & 3;
        int v = QT == QT_Q2B ? s * (2 * c - 3) : s * (c - 1);
        r |= (uint64_t)int_to_op16<F16>(v) << (16 * i);
    }
    return r;
}

template <int QT>
__host__ __device__ constexpr int val_entries() {
    return Fmt<QT>::NSCALE * 256;
}

// ------------------------------------------------------------------ memory sources
// Plain pointer (host tests; device code with a padded buffer).
struct PtrSrc {
    const uint8_t* p;
    __host__ __device__ inline uint32_t dw(uint32_t off) const {
        uint32_t v;
        memcpy(&v, p + off, 4);
        return v;
    }
    __host__ __device__ inline void dw4(uint32_t off, uint32_t o[4]) const {
        for (int i = 0; i < 4; ++i) o[i] = dw(off + 4 * i);
    }
    __host__ __device__ inline void dw2(uint32_t off, uint32_t o[2]) const {
        o[0] = dw(off);
        o[1] = dw(off + 4);
    }
    __host__ __device__ inline void dw3(uint32_t off, uint32_t o[3]) const {
        for (int i = 0; i < 3; ++i) o[i] = dw(off + 4 * i);
    }
    // offset split into a per-lane part and a uniform part (same bytes as dw*(off + soff))
    __host__ __device__ inline uint32_t dw(uint32_t off, uint32_t soff) const { return dw(off + soff); }
    __host__ __device__ inline void dw2(uint32_t off, uint32_t soff, uint32_t o[2]) const { dw2(off + soff, o); }
    __host__ __device__ inline void dw3(uint32_t off, uint32_t soff, uint32_t o[3]) const { dw3(off + soff, o); }
};

// Buffer resource over one matrix of the arena (offsets are bytes from the matrix start; the
// base is 4-byte aligned and the range is rounded up to whole dwords).  Buffer loads at any byte
// offset return the bytes at that offset (gfx950 runs in unaligned access mode).
struct BufSrc {
    __amdgpu_buffer_rsrc_t r;
    __device__ inline BufSrc() {}
    __device__ inline BufSrc(const void* base, uint32_t bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)((bytes + 3u) & ~3u), 0x00020000)) {}
    __device__ inline uint32_t dw(uint32_t off) const { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0); }
    __device__ inline void dw4(uint32_t off, uint32_t o[4]) const {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        o[0] = v[0];
        o[1] = v[1];
        o[2] = v[2];
        o[3] = v[3];
    }
    __device__ inline void dw2(uint32_t off, uint32_t o[2]) const {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        o[0] = v[0];
        o[1] = v[1];
    }
    __device__ inline void dw3(uint32_t off, uint32_t o[3]) const { dw3(off, 0u, o); }
    // per-lane offset `off` plus a wave-uniform offset `soff` (kept in a scalar register)
    __device__ inline uint32_t dw(uint32_t off, uint32_t soff) const {
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0);
    }
    __device__ inline void dw2(uint32_t off, uint32_t soff, uint32_t o[2]) const {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0);
        o[0] = v[0];
        o[1] = v[1];
    }
    __device__ inline void dw3(uint32_t off, uint32_t soff, uint32_t o[3]) const {
        const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, off, soff, 0);
        o[0] = v[0];
        o[1] = v[1];
        o[2] = v[2];
    }
};

// ------------------------------------------------------------------ strips
// STRIP consecutive values (16, 32 or 64) of one row inside one block, starting at value vs
// (a multiple of 8).  Raw dwords: the aligned dwords of the block header and of the strip's
// byte window.
template <int QT, int STRIP>
struct StripRaw {
    static constexpr int HW = Fmt<QT>::HDR_DW;
    static constexpr int WB = QT == QT_Q2B ? STRIP / 4 : (STRIP + 4 + 4) / 5;  // window bytes
    static constexpr int WW = (WB + 3 + 3) / 4;                                // window dwords
    uint32_t h[HW];
    uint32_t w[WW];
    uint32_t hm, wm;  // misalignment (bytes) of header and window
    int vs;

    template <class Src>
    __host__ __device__ inline void load(const Src& src, uint32_t blk_off, int v) {
        vs = v;
        hm = blk_off & 3u;
        const uint32_t ha = blk_off - hm;
        if constexpr (HW == 4)
            src.dw4(ha, h);
        else
            src.dw2(ha, h);
        uint32_t woff;
        if constexpr (QT == QT_Q2B)
            woff = blk_off + 10u + (uint32_t)(v >> 2);
        else
            woff = blk_off + 5u + (uint32_t)(v / 5);
        wm = woff & 3u;
        const uint32_t wa = woff - wm;
        if constexpr (WW >= 4) {
            src.dw4(wa, w);
            if constexpr (WW == 5) w[4] = src.dw(wa + 16);
        } else if constexpr (WW == 3) {
            src.dw2(wa, w);
            w[2] = src.dw(wa + 8);
        } else {
            src.dw2(wa, w);
        }
    }
};

template <int QT, int STRIP>
struct Strip {
    static constexpr int NFRAG = STRIP / 8;
    static constexpr int SW = (STRIP * 2 + 31) / 32;      // dwords of 2-bit codes
    static constexpr int FPS = QT == QT_T1 ? 4 : 2;       // fragments per sub-scale
    static constexpr int NSB = (NFRAG + FPS - 1) / FPS;   // sub-scales the strip touches
    uint32_t code[SW];  // 2-bit codes of values vs..vs+STRIP-1
    uint32_t sb[NSB];   // value-table row (s * 256) of each sub-scale; 0 everywhere when d = 0
    float d;            // block scale applied to the integer dot product

    // vs must be a multiple of min(STRIP, sub-scale span): strips never straddle a sub-scale
    // boundary except at fragment-group boundaries (true for every strip the kernels use).
    __host__ __device__ inline void prepare(const StripRaw<QT, STRIP>& raw, const uint32_t* tern) {
        const int vs = raw.vs;
        const uint32_t h0 = funnel(raw.h[1], raw.h[0], raw.hm);
        if constexpr (QT == QT_Q2B) {
            const uint32_t h1 = funnel(raw.h[2], raw.h[1], raw.hm);
            const uint32_t h2 = funnel(raw.h[3], raw.h[2], raw.hm);
            d = half_bits_to_float(h0 & 0xFFFFu) * 0.5f;
            // scale bytes 2..9 as one 64-bit word: nibble j = sub-scale of values 16j..16j+15
            const uint64_t sw = ((uint64_t)h2 << 48) | ((uint64_t)h1 << 16) | (h0 >> 16);
#pragma unroll
            for (int i = 0; i < NSB; ++i) sb[i] = (uint32_t)((sw >> (4 * ((vs >> 4) + i))) & 15u) << 8;
        } else {
            const uint32_t h1 = funnel(0u, raw.h[1], raw.hm);
            d = half_bits_to_float(h0 & 0xFFFFu);
            const uint32_t sw = (h0 >> 16) | ((h1 & 255u) << 16);
#pragma unroll
            for (int i = 0; i < NSB; ++i) sb[i] = ((sw >> (3 * ((vs >> 5) + i))) & 7u) << 8;
        }
        if (d == 0.0f) {
#pragma unroll
            for (int i = 0; i < NSB; ++i) sb[i] = 0u;  // s = 0 rows of the value table are zero
        }
        constexpr int AW = StripRaw<QT, STRIP>::WW - 1;
        uint32_t a[AW];
#pragma unroll
        for (int i = 0; i < AW; ++i) a[i] = funnel(raw.w[i + 1], raw.w[i], raw.wm);
        if constexpr (QT == QT_Q2B) {
#pragma unroll
            for (int i = 0; i < SW; ++i) code[i] = a[i];
        } else {
            const int b0 = vs / 5;
            const int r = vs - 5 * b0;
            constexpr int NB = StripRaw<QT, STRIP>::WB;
            uint32_t st[SW + 1];
#pragma unroll
            for (int i = 0; i <= SW; ++i) st[i] = 0u;
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const uint32_t c = tern[(a[i >> 2] >> (8 * (i & 3))) & 255u];
                const int bit = 10 * i;
                if (bit / 32 <= SW) st[bit / 32] |= c << (bit % 32);
                if ((bit % 32) > 22 && bit / 32 + 1 <= SW) st[bit / 32 + 1] |= c >> (32 - bit % 32);
            }
#pragma unroll
            for (int i = 0; i < SW; ++i) code[i] = (uint32_t)((((uint64_t)st[i + 1] << 32) | st[i]) >> (2 * r));
        }
    }

    // operand of fragment f (values vs+8f..vs+8f+7); f must be a compile-time constant in
    // kernels so that the code words stay in registers
    __host__ __device__ inline u32x4 frag(int f, const uint64_t* val) const {
        const uint32_t w = code[f >> 1] >> (16 * (f & 1));
        const uint32_t base = sb[f / FPS];
        const uint64_t lo = val[base + (w & 255u)];
        const uint64_t hi = val[base + ((w >> 8) & 255u)];
        u32x4 r;
        r[0] = (uint32_t)lo;
        r[1] = (uint32_t)(lo >> 32);
        r[2] = (uint32_t)hi;
        r[3] = (uint32_t)(hi >> 32);
        return r;
    }

    // the same operand divided by its sub-scale, from the unit row (s = 1) of the value table
    // (val1 = 256 entries); sub(f / FPS) is the factor that restores it
    __host__ __device__ inline u32x4 frag1(int f, const uint64_t* val1) const {
        const uint32_t w = code[f >> 1] >> (16 * (f & 1));
        const uint64_t lo = val1[w & 255u];
        const uint64_t hi = val1[(w >> 8) & 255u];
        u32x4 r;
        r[0] = (uint32_t)lo;
        r[1] = (uint32_t)(lo >> 32);
        r[2] = (uint32_t)hi;
        r[3] = (uint32_t)(hi >> 32);
        return r;
    }
    // sub-scale i of the strip (0 when the block scale is 0)
    __host__ __device__ inline float sub(int i) const { return (float)(sb[i] >> 8); }
};

// ------------------------------------------------------------------ T1 strips for the fp8 MFMA
// The 16x16x128 fp8 MFMA contracts 128 k per step; lane group g (lanes 16g..16g+15) supplies
// 32 bytes of k.  Any bijection between (lane group, operand byte) and k is allowed as long as
// the activation operand uses the same one, so each lane group takes whole digit bytes of a
// 256-value block: over the block's two steps, operand byte j (0..63) of lane group g holds
//   value t1_kmap(g, j) = 60g + j          for j < 60   (digit bytes 12g .. 12g+11)
//                         240 + 4g + j-60  for j >= 60  (four of the 16 values in bytes 48..51)
// and step h takes operand bytes 32h .. 32h+31.
__host__ __device__ constexpr int t1_kmap(int g, int j) { return j < 60 ? 60 * g + j : 240 + 4 * g + (j - 60); }

// Selector table: entry (r, b) holds the five base-3 digits of byte b (least significant first,
// each 0..2) as bytes r .. r+4 of a 64-bit word (r = 0..3).  Bytes above 242 are not produced by
// the format; they decode as five 1-digits (weight 0).
constexpr int TSEL_ENTRIES = 4 * 256;
__host__ __device__ inline uint64_t tsel_entry(int idx) {
    const int r = idx >> 8;
    uint32_t b = (uint32_t)idx & 255u;
    if (b > 242u) b = 121u;  // 11111 in base 3
    uint64_t v = 0;
    for (int i = 0; i < 5; ++i) {
        v |= (uint64_t)(b % 3u) << (8 * (i + r));
        b /= 3u;
    }
    return v;
}

// Raw bytes of one lane's share of a T1 block: bytes 0..7 (d, sub-scales; byte 4 in the low
// byte of h[1]), the 12 digit bytes 12g.. of the lane group, and the block's last four bytes
// (digit bytes 48..51).  They are cut out of a 64-byte window of dwords that starts at the
// dword boundary at or below the block start (m = block start % 4), which holds the whole
// 57-byte block; kernels fetch such windows with coalesced loads (four lanes per row).
struct T1Raw8 {
    uint32_t h[2], w[3], t;
    template <class Win>
    __host__ __device__ inline void load_window(const Win& win, uint32_t m, int g) {
        const uint32_t h0 = win[0], h1 = win[1];
        h[0] = funnel(h1, h0, m);
        h[1] = h1 >> (8u * m);
        const uint32_t o = m + 5u + 12u * (uint32_t)g, d = o >> 2, s = o & 3u;
        const uint32_t w0 = win[d], w1 = win[d + 1], w2 = win[d + 2], w3 = win[d + 3];
        w[0] = funnel(w1, w0, s);
        w[1] = funnel(w2, w1, s);
        w[2] = funnel(w3, w2, s);
        const uint32_t o2 = m + 53u, d2 = o2 >> 2, s2 = o2 & 3u;
        t = funnel(win[d2 + 1], win[d2], s2);
    }
};

// Per-lane constants of lane group g.
struct T1Lane8 {
    uint32_t shA, shB, shC;      // bit position of the sub-scales used by the lane (3 per group)
    uint32_t m1, m2, m8, m9, m10;  // +4 on the selectors of dwords that take the second table
    uint32_t tbs;                // tail: first tail byte 48 + (4g)/5 as a bit shift of the last dword
    uint32_t tsh;                // tail: digit offset inside its first byte, in bits
    uint32_t trot, tmask;        // tail: rotation of the second byte's lookup, and its mask
    __host__ __device__ inline void init(int g) {
        // dword q (values 60g+4q .. +3) lies in sub-scale group (60g+4q)/32: groups
        // A = max(2g-1, 0), B = 2g, C = 2g+1 cover every lane (for g = 0, A = B)
        shA = 3u * (uint32_t)(g > 0 ? 2 * g - 1 : 0);
        shB = 3u * (uint32_t)(2 * g);
        shC = 3u * (uint32_t)(2 * g + 1);
        const uint32_t M = 0x04040404u;
        m1 = g == 1 ? M : 0u;
        m2 = (g == 1 || g == 2) ? M : 0u;
        m8 = g == 0 ? M : 0u;
        m9 = g <= 1 ? M : 0u;
        m10 = g <= 2 ? M : 0u;
        const int r0 = (4 * g) % 5;
        tbs = 8u * (uint32_t)((4 * g) / 5);
        tsh = 8u * (uint32_t)r0;
        trot = r0 == 0 ? 0u : (uint32_t)(5 - r0);
        tmask = r0 == 0 ? 0u : 0xFFFFFFFFu;
    }
};

// Decoder of one lane's share of a T1 block, in two parts so that a kernel holds the operands
// of one MFMA step at a time: prep() takes the raw dwords (which can then be reused for the
// next block's loads) and keeps the aligned digit bytes, the tail word and the four scale
// tables; step(h, ...) returns the fp8 operand of step h (exact s*(digit-1)).
// tbl8[s] = [e(-s), e(0), e(+s), 0] (e = the fp8 e4m3 encoding; all zero for s = 0).  A block
// with d = 0 decodes to zero operands.
struct T1Dec8 {
    uint32_t a[3];              // digit bytes 12g .. 12g+11 of the lane group
    uint32_t tw;                // tail bytes 48 + (4g)/5 and the next one (low 16 bits)
    uint32_t TA, TB, TC, TD;    // scale tables of the lane's sub-scale groups (see T1Lane8), TD: group 7
    float d;

    // live = false: a padding block, decoded as zero (d = 0)
    __host__ __device__ inline void prep(const T1Raw8& raw, const T1Lane8& ln, const uint32_t* tbl8,
                                         bool live = true) {
        d = live ? half_bits_to_float(raw.h[0] & 0xFFFFu) : 0.0f;  // (live = false: a block of zeros)
        uint32_t sw = (raw.h[0] >> 16) | (raw.h[1] << 16);  // bits 3i..3i+2: sub-scale of values 32i..32i+31
        if (d == 0.0f) sw = 0u;
        TA = tbl8[(sw >> ln.shA) & 7u];
        TB = tbl8[(sw >> ln.shB) & 7u];
        TC = tbl8[(sw >> ln.shC) & 7u];
        TD = tbl8[(sw >> 21) & 7u];
#pragma unroll
        for (int i = 0; i < 3; ++i) a[i] = raw.w[i];
        tw = raw.t >> ln.tbs;
    }

    // selector entry of digit byte j (0..11) with rotation j%4: covers stream dwords
    // 5(j/4) + j%4 and the next one
    __host__ __device__ inline uint64_t sel(int j, const uint64_t* tsel) const {
        return tsel[(j & 3) * 256 + ((a[j >> 2] >> (8 * (j & 3))) & 255u)];
    }

    // the selector entries that step h needs (h = 0: bytes 0..6; h = 1: bytes 6..11 and the
    // two tail entries), issued apart from their use so that a kernel can overlap the lookups
    // with other work
    __host__ __device__ inline void look(int h, const T1Lane8& ln, const uint64_t* tsel, uint64_t e[8]) const {
        if (h == 0) {
#pragma unroll
            for (int j = 0; j < 7; ++j) e[j] = sel(j, tsel);
            e[7] = 0;
        } else {
#pragma unroll
            for (int j = 6; j < 12; ++j) e[j - 6] = sel(j, tsel);
            e[6] = tsel[tw & 255u];
            e[7] = tsel[ln.trot * 256u + ((tw >> 8) & 255u)];
        }
    }

    // the fp8 operand of step h from its selector entries
    __host__ __device__ inline void build(int h, const T1Lane8& ln, const uint64_t e[8], uint32_t b[8]) const {
        // stream dwords of groups of four bytes: q[5m] = lo(4m), q[5m+1..3] = hi | lo, q[5m+4] = hi(4m+3)
        uint32_t lo[8], hi[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            lo[j] = (uint32_t)e[j];
            hi[j] = (uint32_t)(e[j] >> 32);
        }
        if (h == 0) {  // stream dwords 0..7: bytes 0..6
            const uint32_t q0 = lo[0], q1 = hi[0] | lo[1] | ln.m1, q2 = hi[1] | lo[2] | ln.m2;
            const uint32_t q3 = hi[2] | lo[3], q4 = hi[3], q5 = lo[4], q6 = hi[4] | lo[5], q7 = hi[5] | lo[6];
            // selectors 0..3 pick from the first table, 4..7 from the second
            b[0] = perm2(TA, TA, q0);
            b[1] = perm2(TB, TA, q1);
            b[2] = perm2(TB, TA, q2);
            b[3] = perm2(TB, TB, q3);
            b[4] = perm2(TB, TB, q4);
            b[5] = perm2(TB, TB, q5);
            b[6] = perm2(TB, TB, q6);
            b[7] = perm2(TB, TB, q7);
        } else {  // stream dwords 8..14: bytes 6..11 (entries 0..5), dword 15: tail (entries 6, 7)
            const uint32_t q8 = hi[0] | lo[1] | ln.m8, q9 = hi[1] | ln.m9, q10 = lo[2] | ln.m10;
            const uint32_t q11 = hi[2] | lo[3], q12 = hi[3] | lo[4], q13 = hi[4] | lo[5], q14 = hi[5];
            const uint32_t q15 = (uint32_t)(e[6] >> ln.tsh) | (lo[7] & ln.tmask);
            b[0] = perm2(TC, TB, q8);
            b[1] = perm2(TC, TB, q9);
            b[2] = perm2(TC, TB, q10);
            b[3] = perm2(TC, TC, q11);
            b[4] = perm2(TC, TC, q12);
            b[5] = perm2(TC, TC, q13);
            b[6] = perm2(TC, TC, q14);
            b[7] = perm2(TD, TD, q15);
        }
    }

    __host__ __device__ inline void step(int h, const T1Lane8& ln, const uint64_t* tsel, uint32_t b[8]) const {
        uint64_t e[8];
        look(h, ln, tsel, e);
        build(h, ln, e, b);
    }
};

// ------------------------------------------------------------------ Q2B strips for the 16-bit MFMA
// The 16x16x32 bf16/fp16 MFMA contracts 32 k per instruction, 8 per lane group.  A 256-value
// Q2B block takes two steps of four MFMAs, and lane group g owns the 64 consecutive values
// 64g .. 64g+63 (code bytes 16g .. 16g+15, sub-scales 4g .. 4g+3): operand j (0..3) of step h
// holds values 64g + 32h + 8j .. +7 in order, two per dword (the lower value in the low half).
// The activations use the same order, which for them is plain row order in 16-byte pieces.
__host__ __device__ constexpr int q2_kmap(int g, int h, int j, int i) { return 64 * g + 32 * h + 8 * j + i; }

// Selector table: entry b (a byte of four 2-bit codes c0..c3, c0 in the low bits) holds the
// v_perm selectors that pick the 16-bit operands of (c0, c1) [low dword] and (c2, c3) [high
// dword] from an 8-byte value row in which code c's operand sits at bytes 2c, 2c+1.
constexpr int QSEL_ENTRIES = 256;
__host__ __device__ inline uint64_t qsel_entry(int b) {
    uint64_t v = 0;
    for (int i = 0; i < 4; ++i) {
        const uint64_t c = ((uint32_t)b >> (2 * i)) & 3u;
        v |= (2 * c) << (16 * i);
        v |= (2 * c + 1) << (16 * i + 8);
    }
    return v;
}

// Value row of sub-scale s (0..15): the 16-bit operands s*(2c - 3), c = 0..3, exact in bf16 and fp16.
constexpr int Q2ROW_ENTRIES = 16;
template <bool F16>
__host__ __device__ inline uint64_t q2row_entry(int s) {
    uint64_t v = 0;
    for (int c = 0; c < 4; ++c) v |= (uint64_t)int_to_op16<F16>(s * (2 * c - 3)) << (16 * c);
    return v;
}

// Raw bytes of one lane's share of a Q2B block (d, the two scale bytes of its sub-scales, its 16
// code bytes), cut out of an 80-byte window of dwords that starts at the dword boundary at or
// below the block start (m = block start % 4); the window holds the whole 74-byte block.
struct Q2Raw16 {
    uint32_t h;     // low 16 bits: d
    uint32_t sc;    // low 16 bits: scale bytes 2+2g and 3+2g
    uint32_t c[4];  // code bytes 16g .. 16g+15
    template <class Win>
    __host__ __device__ inline void load_window(const Win& win, uint32_t m, int g) {
        h = funnel(win[1], win[0], m);
        const uint32_t os = m + 2u + 2u * (uint32_t)g, ds = os >> 2, ss = os & 3u;
        sc = funnel(win[ds + 1], win[ds], ss);
        const uint32_t o = m + 10u + 16u * (uint32_t)g, d = o >> 2, s = o & 3u;
        const uint32_t w0 = win[d], w1 = win[d + 1], w2 = win[d + 2], w3 = win[d + 3], w4 = win[d + 4];
        c[0] = funnel(w1, w0, s);
        c[1] = funnel(w2, w1, s);
        c[2] = funnel(w3, w2, s);
        c[3] = funnel(w4, w3, s);
    }
};

// Decoder of one lane's share of a Q2B block: prep() keeps the code bytes and the value rows of
// the lane's four sub-scales; half(h, p, ...) returns operands 2p and 2p+1 of step h (8 dwords),
// so that a kernel holds half a step's operands at a time.  d is the block scale of the integer
// dot products (half the fp16 d, as s*(2c - 3) = 2*s*(c - 1.5)).  A block with d = 0 decodes to
// zero operands.
struct Q2Dec16 {
    uint32_t c[4];
    uint32_t TL[4], TH[4];  // value row of sub-scale 4g+i: operands of codes 0, 1 | 2, 3
    float d;
    __host__ __device__ inline void prep(const Q2Raw16& raw, const uint64_t* q2row, bool live = true) {
        d = live ? half_bits_to_float(raw.h & 0xFFFFu) * 0.5f : 0.0f;
        uint32_t sw = raw.sc & 0xFFFFu;  // nibble i: sub-scale 4g+i
        if (d == 0.0f) sw = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint64_t r = q2row[(sw >> (4 * i)) & 15u];
            TL[i] = (uint32_t)r;
            TH[i] = (uint32_t)(r >> 32);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = raw.c[i];
    }
    __host__ __device__ inline void half(int h, int p, const uint64_t* qsel, uint32_t b[8]) const {
        const int sb = 2 * h + p;  // operands 2p, 2p+1 of step h: values 32h + 16p .. +15, one sub-scale
        const uint32_t w = c[sb];
        const uint32_t tl = TL[sb], th = TH[sb];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint64_t e = qsel[(w >> (8 * i)) & 255u];
            b[2 * i] = perm2(th, tl, (uint32_t)e);
            b[2 * i + 1] = perm2(th, tl, (uint32_t)(e >> 32));
        }
    }
};

}  // namespace rl
