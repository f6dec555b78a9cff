// K-tail kernels of table row 8 (see mg_table.h).
#include "mg_launch.h"

MG_DEFINE_ROW_TAIL(8, Fast8)
