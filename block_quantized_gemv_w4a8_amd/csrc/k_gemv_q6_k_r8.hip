// k_gemv_q6_k_r8.hip -- the Q6_K_R8 GEMV launchers (kernel templates in k_gemv.h).
#include "k_gemv.h"

namespace qgemv {

QGEMV_GEMV_FORMAT_ENTRIES(q6_k_r8, QGEMV_FMT_Q6_K_R8)

}  // namespace qgemv
