// k_gemv_q8_0.hip -- the Q8_0 GEMV launchers (kernel templates in k_gemv.h).
#include "k_gemv.h"

namespace qgemv {

QGEMV_GEMV_FORMAT_ENTRIES(q8_0, QGEMV_FMT_Q8_0)

}  // namespace qgemv
