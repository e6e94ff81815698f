// Host-side packing between the canonical MLX-affine layout and DEV_V1.
// Every code, scale and bias is copied unchanged; only positions move.
// DEV_V1 keeps one (scale, bias) pair per row and 64-column block, so a
// matrix quantized in groups of 64 n columns is packed with each group's
// pair copied into its n blocks: the same weights, w = s q + b, and the
// exact inverse collapses the copies again.
#include <string.h>

#include "../../include/moegemv.h"
#include "layout.h"

using namespace mq;

static bool group_ok(int32_t cols, int32_t group) {
    return group > 0 && group % kGroup == 0 && cols > 0 && cols % group == 0;
}

extern "C" size_t mq_packed_bytes(int32_t rows, int32_t cols, int32_t bits, int32_t group, int32_t layout) {
    if (rows <= 0 || cols <= 0 || !group_ok(cols, group) || (bits != 4 && bits != 8)) return 0;
    if (layout == MQ_LAYOUT_CANONICAL)
        return (size_t)rows * cols * bits / 8 + (size_t)rows * (cols / group) * 4;
    if (layout == MQ_LAYOUT_DEV_V1)
        return (size_t)(pad_rows(rows) / kTileRows) * (cols / kGroup) * blk_bytes(bits);
    return 0;
}

extern "C" int64_t mq_pool_layout(int32_t hidden, int32_t inter, int32_t bits, int32_t group,
                                  int64_t page_bytes, mq_expert_pool* pool) {
    if (!pool || page_bytes < 256 || (page_bytes & (page_bytes - 1))) return 0;
    size_t gu = mq_packed_bytes(inter, hidden, bits, group, MQ_LAYOUT_DEV_V1);
    size_t dn = mq_packed_bytes(hidden, inter, bits, group, MQ_LAYOUT_DEV_V1);
    if (!gu || !dn) return 0;
    int64_t blob = (int64_t)(2 * gu + dn);
    int64_t stride = (blob + page_bytes - 1) / page_bytes * page_bytes;
    pool->gate_offset = 0;
    pool->up_offset = (int64_t)gu;
    pool->down_offset = (int64_t)(2 * gu);
    pool->expert_stride = stride;
    pool->hidden = hidden;
    pool->inter = inter;
    pool->bits = bits;
    pool->group = group;
    pool->layout = MQ_LAYOUT_DEV_V1;
    return stride;
}

static bool tensor_ok(const mq_qtensor* t) {
    return t && t->rows > 0 && group_ok(t->cols, t->group) && (t->bits == 4 || t->bits == 8);
}

// Row and first column of word (j, lane, i) of a block (see include/moegemv.h).
static inline void word_origin(int bits, int j, int lane, int i, int* row, int* col) {
    int a = 4 * j + i;
    if (bits == 4) {
        *row = 16 * (a >> 1) + (lane & 15);
        *col = 32 * (a & 1) + 8 * (lane >> 4);
    } else {
        *row = 16 * (a >> 2) + (lane & 15);
        *col = 16 * (a & 3) + 4 * (lane >> 4);
    }
}

extern "C" mq_status mq_pack(const mq_qtensor* src, void* dst, size_t dst_bytes, mq_qtensor* dst_desc) {
    if (!src || !dst || !src->codes || !src->scales || !src->biases) return MQ_ERR_NULL;
    if (!tensor_ok(src)) return MQ_ERR_UNSUPPORTED;
    if (src->layout != MQ_LAYOUT_CANONICAL) return MQ_ERR_UNSUPPORTED;
    size_t need = mq_packed_bytes(src->rows, src->cols, src->bits, src->group, MQ_LAYOUT_DEV_V1);
    if (dst_bytes < need) return MQ_ERR_BUFFER;
    const int bits = src->bits, G = src->cols / kGroup, Gs = src->cols / src->group, per = src->group / kGroup;
    const int64_t wpr = (int64_t)src->cols * bits / 32;     // canonical words per row
    const uint32_t* cw = (const uint32_t*)src->codes;
    const uint16_t* sc = (const uint16_t*)src->scales;
    const uint16_t* bi = (const uint16_t*)src->biases;
    const int tiles = (int)(pad_rows(src->rows) / kTileRows);
    const int jn = bits == 4 ? 2 : 4;
    const int cols_per_word = 32 / bits;
    uint8_t* out = (uint8_t*)dst;
    for (int t = 0; t < tiles; ++t) {
        for (int g = 0; g < G; ++g) {
            uint8_t* blk = out + ((int64_t)t * G + g) * blk_bytes(bits);
            uint32_t* wd = (uint32_t*)blk;
            for (int j = 0; j < jn; ++j)
                for (int lane = 0; lane < 64; ++lane)
                    for (int i = 0; i < 4; ++i) {
                        int r, c;
                        word_origin(bits, j, lane, i, &r, &c);
                        int64_t row = (int64_t)t * kTileRows + r;
                        uint32_t w = 0;
                        if (row < src->rows) {
                            w = cw[row * wpr + (g * kGroup + c) / cols_per_word];
                            if (bits == 4) w = nib_to_dev(w);
                        }
                        wd[(j * 64 + lane) * 4 + i] = w;
                    }
            uint32_t* sb = (uint32_t*)(blk + code_bytes(bits));
            for (int r = 0; r < 16; ++r)
                for (int m = 0; m < 4; ++m) {
                    int64_t row = (int64_t)t * kTileRows + 16 * m + r;
                    uint32_t v = 0;
                    if (row < src->rows)
                        v = (uint32_t)sc[row * Gs + g / per] | ((uint32_t)bi[row * Gs + g / per] << 16);
                    sb[r * 4 + m] = v;
                }
        }
    }
    if (dst_desc) {
        *dst_desc = *src;
        dst_desc->codes = dst;
        dst_desc->scales = nullptr;
        dst_desc->biases = nullptr;
        dst_desc->layout = MQ_LAYOUT_DEV_V1;
    }
    return MQ_OK;
}

extern "C" mq_status mq_unpack(const mq_qtensor* src, uint32_t* codes, uint16_t* scales, uint16_t* biases) {
    if (!src || !src->codes || !codes || !scales || !biases) return MQ_ERR_NULL;
    if (!tensor_ok(src)) return MQ_ERR_UNSUPPORTED;
    if (src->layout != MQ_LAYOUT_DEV_V1) return MQ_ERR_UNSUPPORTED;
    const int bits = src->bits, G = src->cols / kGroup, Gs = src->cols / src->group, per = src->group / kGroup;
    const int64_t wpr = (int64_t)src->cols * bits / 32;
    const int tiles = (int)(pad_rows(src->rows) / kTileRows);
    const int jn = bits == 4 ? 2 : 4;
    const int cols_per_word = 32 / bits;
    const uint8_t* in = (const uint8_t*)src->codes;
    // a group of 64 n columns holds one pair: every block of it must carry the
    // same pair, or the region is not a tensor of that group size
    if (per > 1)
        for (int t = 0; t < tiles; ++t)
            for (int g = 0; g < G; ++g) {
                const uint32_t* sb = (const uint32_t*)(in + ((int64_t)t * G + g) * blk_bytes(bits) + code_bytes(bits));
                const uint32_t* s0 =
                    (const uint32_t*)(in + ((int64_t)t * G + g / per * per) * blk_bytes(bits) + code_bytes(bits));
                for (int q = 0; q < 64; ++q)
                    if (sb[q] != s0[q]) return MQ_ERR_UNSUPPORTED;
            }
    for (int t = 0; t < tiles; ++t) {
        for (int g = 0; g < G; ++g) {
            const uint8_t* blk = in + ((int64_t)t * G + g) * blk_bytes(bits);
            const uint32_t* wd = (const uint32_t*)blk;
            for (int j = 0; j < jn; ++j)
                for (int lane = 0; lane < 64; ++lane)
                    for (int i = 0; i < 4; ++i) {
                        int r, c;
                        word_origin(bits, j, lane, i, &r, &c);
                        int64_t row = (int64_t)t * kTileRows + r;
                        if (row >= src->rows) continue;
                        uint32_t w = wd[(j * 64 + lane) * 4 + i];
                        if (bits == 4) w = nib_from_dev(w);
                        codes[row * wpr + (g * kGroup + c) / cols_per_word] = w;
                    }
            const uint32_t* sb = (const uint32_t*)(blk + code_bytes(bits));
            for (int r = 0; r < 16; ++r)
                for (int m = 0; m < 4; ++m) {
                    int64_t row = (int64_t)t * kTileRows + 16 * m + r;
                    if (row >= src->rows) continue;
                    uint32_t v = sb[r * 4 + m];
                    scales[row * Gs + g / per] = (uint16_t)(v & 0xFFFFu);
                    biases[row * Gs + g / per] = (uint16_t)(v >> 16);
                }
        }
    }
    return MQ_OK;
}
