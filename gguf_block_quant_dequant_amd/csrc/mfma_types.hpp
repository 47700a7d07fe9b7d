// Operand and accumulator vectors of the gfx950 bf16 matrix instruction
// v_mfma_f32_32x32x16_bf16 (8 bf16 of A or B per lane, 16 fp32 of D per lane).
#pragma once

namespace gqk {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

}  // namespace gqk
