// K-tail kernels of table row 3 (see mg_table.h).
#include "mg_launch.h"

MG_DEFINE_ROW_TAIL(3, Fast3)
